// Induced-subgraph build: one bit-encoded table per first-level subtree root,
// written into a shared HBM heap before the search launch that uses it.
//
// "Parallelizing Maximal Clique Enumeration on GPUs" (arxiv 2212.01473v2):
//  - section 2.4 (induced subgraphs): a subtree only needs the edges between
//    P u X and P, where P / X are the root's later / earlier neighbours;
//  - section 3.4: binary-encoded rows; the full subgraph holds rows for every
//    vertex of P u X over P, the partial one rows for P over P only (P-X edges
//    are then looked up in the CSR during the search).
//
// Table layout (u64 words, see mce_table_words; micro tables add the X column of
// every P member after the rows, see mce_micro_table_words): header (p | x << 32), root id,
// root hash term, rows (row a = bit b set iff L[a] ~ P[b], local order = id
// order, P first), p hash terms of the P members, p + x int32 ids.
//
// One 64-lane wavefront per root. A row is filled either by streaming the
// member's CSR row and looking every neighbour up in P (sorted, in LDS), or, for
// members of high degree, by probing each P member in that CSR row.
#include "mce_device.h"
#include "mce_internal.h"

__global__ __launch_bounds__(64) void k_build(BuildParams prm) {
  __shared__ int s_pid[MCE_MAX_P];
  __shared__ u64 s_row[MCE_MAX_P / 64];
  const int lane = lane_id();
  const int W = prm.W;
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ ci = prm.ci;
  const int* __restrict__ rnd = prm.rnd;
  for (int i = blockIdx.x; i < prm.nroots; i += gridDim.x) {
    const int r = prm.roots[i];
    const int a = rp[r], b = rp[r + 1];
    const int rr = rnd[r];
    // P = later neighbours into LDS (ascending id); count X
    int np = 0, nx = 0;
    for (int base = a; base < b; base += MCE_WAVE) {
      const int e = base + lane;
      const bool valid = e < b;
      const int u = valid ? ci[e] : 0;
      const bool lat = valid && order_after(rnd[u], u, rr, r);
      const u64 lm = ballot(lat);
      const u64 xm = ballot(valid && !lat);
      if (lat) {
        const int pos = np + mbcnt(lm);
        if (pos < MCE_MAX_P) s_pid[pos] = u;
      }
      np += __popcll(lm);
      nx += __popcll(xm);
    }
    if (np == 0 || np > 64 * W) {   // the host only sends 1 <= |P| <= 64 W here
      if (lane == 0) {
        atomicOr(prm.status, MCE_E_LIMIT);
        prm.tab_off[i] = 0;
      }
      continue;
    }
    const long long nrows = mce_table_rows(np, nx, prm.micro ? MCE_MODE_IPX : prm.mode);
    const u64 words = prm.micro ? mce_micro_table_words(np, nx) : mce_table_words(np, nx, W, prm.mode);
    u64 off = 0;
    if (lane == 0) off = atomicAdd(prm.heap_top, words);
    off = read_lane(off, 0);
    if (off + words > prm.heap_words) {
      if (lane == 0) {
        atomicOr(prm.status, MCE_E_HEAP);
        prm.tab_off[i] = 0;
      }
      continue;
    }
    if (lane == 0) prm.tab_off[i] = off;
    u64* T = prm.heap + off;
    u64* rows = T + 3;
    u64* xcol = rows + (size_t)nrows * W;   // micro tables only
    u64* hvs = prm.micro ? xcol + np : xcol;
    int* ids = (int*)(hvs + np);
    if (lane == 0) {
      T[0] = (u64)(u32)np | ((u64)(u32)nx << 32);
      T[1] = (u64)(u32)r;
      T[2] = mce_vertex_term(r);
    }
    __syncthreads();   // s_pid complete
    for (int j = lane; j < np; j += MCE_WAVE) {
      const int g = s_pid[j];
      ids[j] = g;
      hvs[j] = mce_vertex_term(g);
    }
    int xo = 0;
    for (int base = a; base < b; base += MCE_WAVE) {
      const int e = base + lane;
      const bool valid = e < b;
      const int u = valid ? ci[e] : 0;
      const bool ear = valid && !order_after(rnd[u], u, rr, r);
      const u64 xm = ballot(ear);
      if (ear) ids[np + xo + mbcnt(xm)] = u;
      xo += __popcll(xm);
    }
    __syncthreads();   // X ids in the table before the rows read them back
    for (long long ra = 0; ra < nrows; ra++) {
      const int g = ra < np ? s_pid[ra] : ids[ra];
      const int ga = rp[g], gb = rp[g + 1];
      const int gdeg = gb - ga;
      if (gdeg <= 128 * W) {
        // stream N(g) and look every neighbour up in P
        if (lane < W) s_row[lane] = 0;
        __syncthreads();
        for (int base = ga; base < gb; base += MCE_WAVE) {
          const int e = base + lane;
          if (e < gb) {
            const int u = ci[e];
            int lo = 0, len = np;
            while (len > 0) {
              const int half = len >> 1;
              if (s_pid[lo + half] < u) {
                lo += half + 1;
                len -= half + 1;
              } else {
                len = half;
              }
            }
            if (lo < np && s_pid[lo] == u) atomicOr(&s_row[lo >> 6], 1ull << (lo & 63));
          }
        }
        __syncthreads();
        if (lane < W) rows[(size_t)ra * W + lane] = s_row[lane];
        __syncthreads();
      } else {
        // probe every P member in N(g)
        for (int w = 0; w < W; w++) {
          const int j = w * 64 + lane;
          const bool bit = j < np && j != ra && csr_range_has(ci, ga, gb, s_pid[j]);
          const u64 word = ballot(bit);
          if (lane == 0) rows[(size_t)ra * W + w] = word;
        }
      }
    }
    if (prm.micro) {
      // micro table: X column of every P member (the transpose of the X rows)
      __syncthreads();   // the X rows are in the table
      u64 col = 0;
      if (lane < np) {
        for (int j = 0; j < nx; j++) col |= ((rows[np + j] >> lane) & 1ull) << j;
        xcol[lane] = col;
      }
    }
    __syncthreads();
  }
}

hipError_t mce_launch_build(const BuildParams& prm, int blocks, hipStream_t s) {
  const int nb = std::max(1, std::min(blocks, prm.nroots));
  hipLaunchKernelGGL(k_build, dim3(nb), dim3(64), 0, s, prm);
  return hipGetLastError();
}
