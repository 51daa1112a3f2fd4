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
      if (lane == 0) atomicOr(prm.status, MCE_E_LIMIT);
      continue;
    }
    const long long nrows = mce_table_rows(np, nx, prm.micro ? MCE_MODE_IPX : prm.mode);
    const u64 words = prm.micro ? mce_micro_table_words(np, nx) : mce_table_words(np, nx, W, prm.mode);
    const u64 off = uni(prm.tab_off[i]) - uni(prm.tab_off[0]);
    if (off + words > prm.heap_words) {
      if (lane == 0) atomicOr(prm.status, MCE_E_HEAP);
      continue;
    }
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

// ------------------------------------------------------------------ narrow tables
// Tables of |P| <= 64 W for W <= 4 (every micro table, and the narrow width
// classes): one wavefront per root, one lane per row. P's ids go into an LDS
// hash table (key = vertex id, value = local index), so a lane builds its row
// by walking its vertex's CSR row and looking every neighbour up, all rows of a
// 64-row slab at once; rows longer than BUILD_LANE_MAX edges are built instead
// by probing each P member in that CSR row (binary search), one lane per P
// member, several rows per pass when |P| is small.
#define BUILD_LANE_MAX 48

template <int HB>
__device__ __forceinline__ u32 build_hash(int u) {
  return ((u32)u * 0x9E3779B1u) >> (32 - HB);
}

template <int HB>
__device__ __forceinline__ int build_lookup(const int* hk, const short* hv, int u) {
  u32 h = build_hash<HB>(u);
  for (int i = 0; i < (1 << HB); i++) {
    const int k = hk[h];
    if (k == u) return hv[h];
    if (k < 0) return -1;
    h = (h + 1u) & ((1u << HB) - 1u);
  }
  return -1;
}

template <int W>
__global__ __launch_bounds__(64) void k_build_narrow(BuildParams prm) {
  constexpr int PMAX = 64 * W;
  constexpr int HB = W == 1 ? 7 : (W == 2 ? 8 : 9);   // hash slots >= 2 PMAX
  __shared__ int s_pid[PMAX];
  __shared__ int s_hk[1 << HB];
  __shared__ short s_hv[1 << HB];
  __shared__ int s_long[MCE_WAVE];   // rows of the current slab that are built by probing
  __shared__ int s_nlong;
  const int lane = lane_id();
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ ci = prm.ci;
  const int* __restrict__ rnd = prm.rnd;
  const bool micro = prm.micro != 0;
  const int mode = micro ? MCE_MODE_IPX : prm.mode;
  for (int i = blockIdx.x; i < prm.nroots; i += gridDim.x) {
    const int r = prm.roots[i];
    const int a = rp[r], b = rp[r + 1];
    const int rr = rnd[r];
    // P (later neighbours) into LDS, in id order; count X
    int np = 0, nx = 0;
    for (int base = a; base < b; base += MCE_WAVE) {
      const int e = base + lane;
      const bool valid = e < b;
      const int u = valid ? ci[e] : 0;
      const bool lat = valid && order_after(rnd[u], u, rr, r);
      const u64 lm = ballot(lat), xm = ballot(valid && !lat);
      if (lat && np + mbcnt(lm) < PMAX) s_pid[np + mbcnt(lm)] = u;
      np += __popcll(lm);
      nx += __popcll(xm);
    }
    if (np == 0 || np > PMAX || (micro && nx > MCE_MICRO_MAX)) {   // the host sends only such roots here
      if (lane == 0) atomicOr(prm.status, MCE_E_LIMIT);
      continue;
    }
    const int nrows = (int)mce_table_rows(np, nx, mode);
    const u64 words = micro ? mce_micro_table_words(np, nx) : mce_table_words(np, nx, W, mode);
    const u64 off = uni(prm.tab_off[i]) - uni(prm.tab_off[0]);
    if (off + words > prm.heap_words) {
      if (lane == 0) atomicOr(prm.status, MCE_E_HEAP);
      continue;
    }
    u64* T = prm.heap + off;
    u64* rows = T + 3;
    u64* xcol = rows + (size_t)nrows * W;   // micro tables only
    u64* hvs = micro ? xcol + np : xcol;
    int* ids = (int*)(hvs + np);
    if (lane == 0) {
      T[0] = (u64)(u32)np | ((u64)(u32)nx << 32);
      T[1] = (u64)(u32)r;
      T[2] = mce_vertex_term(r);
    }
    // X ids straight into the table (rows read them back)
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
    // hash of P: id -> local index
    for (int h = lane; h < (1 << HB); h += MCE_WAVE) s_hk[h] = -1;
    __syncthreads();
    for (int j = lane; j < np; j += MCE_WAVE) {
      const int u = s_pid[j];
      ids[j] = u;
      hvs[j] = mce_vertex_term(u);
      u32 h = build_hash<HB>(u);
      while (atomicCAS(&s_hk[h], -1, u) != -1) h = (h + 1u) & ((1u << HB) - 1u);
      s_hv[h] = (short)j;
    }
    __syncthreads();   // hash complete, X ids in the table
    // rows, a slab of 64 at a time
    for (int t0 = 0; t0 < nrows; t0 += MCE_WAVE) {
      const int t = t0 + lane;
      if (lane == 0) s_nlong = 0;
      __syncthreads();
      if (t < nrows) {
        const int g = t < np ? s_pid[t] : ids[t];   // X member t - np sits at ids[t]
        const int ga = rp[g], gb = rp[g + 1];
        if (gb - ga > BUILD_LANE_MAX) {
          s_long[atomicAdd(&s_nlong, 1)] = t;
        } else {
          u64 w[W];
#pragma unroll
          for (int q = 0; q < W; q++) w[q] = 0;
          for (int e = ga; e < gb; e += 4) {
            int j[4];
#pragma unroll
            for (int z = 0; z < 4; z++) {
              const int u = e + z < gb ? ci[e + z] : -1;
              j[z] = u >= 0 ? build_lookup<HB>(s_hk, s_hv, u) : -1;
            }
#pragma unroll
            for (int z = 0; z < 4; z++) {
#pragma unroll
              for (int q = 0; q < W; q++)
                if (j[z] >= 64 * q && j[z] < 64 * (q + 1)) w[q] |= 1ull << (j[z] - 64 * q);
            }
          }
#pragma unroll
          for (int q = 0; q < W; q++) rows[(size_t)t * W + q] = w[q];
        }
      }
      __syncthreads();
      // long rows: lane = P member (several rows per pass when |P| is small)
      const int nl = s_nlong;
      const int npw = np <= 1 ? 1 : (np >= 64 ? 64 : 1 << (32 - __builtin_clz((u32)(np - 1))));
      const int per = MCE_WAVE / npw;   // rows per pass (1 when |P| > 32)
      for (int l0 = 0; l0 < nl; l0 += per) {
        const int q = lane / npw, jj = lane % npw;
        const int tq = l0 + q < nl ? s_long[l0 + q] : -1;
        int g = 0, ga = 0, gb = 0;
        if (tq >= 0) {
          g = tq < np ? s_pid[tq] : ids[tq];
          ga = rp[g];
          gb = rp[g + 1];
        }
        for (int w0 = 0; w0 < W; w0++) {
          const int j = w0 * 64 + jj;
          const bool found = tq >= 0 && j < np && csr_range_has(ci, ga, gb, s_pid[j]);
          const u64 fm = ballot(found);
          if (jj == 0 && tq >= 0) {
            const u64 mask = npw >= 64 ? ~0ull : ((1ull << npw) - 1ull);
            rows[(size_t)tq * W + w0] = (fm >> (q * npw)) & mask;
          }
        }
      }
    }
    if (micro) {
      // X column of every P member: the X rows' bit of that member
      __syncthreads();   // the X rows are in the table
      if (lane < np) {
        u64 col = 0;
        for (int x2 = 0; x2 < nx; x2++) col |= ((rows[np + x2] >> lane) & 1ull) << x2;
        xcol[lane] = col;
      }
    }
    __syncthreads();
  }
}

hipError_t mce_launch_build(const BuildParams& prm, int blocks, hipStream_t s) {
  const int nb = std::max(1, std::min(blocks, prm.nroots));
  if (prm.micro || prm.W == 1)
    hipLaunchKernelGGL(k_build_narrow<1>, dim3(nb), dim3(64), 0, s, prm);
  else if (prm.W == 2)
    hipLaunchKernelGGL(k_build_narrow<2>, dim3(nb), dim3(64), 0, s, prm);
  else if (prm.W == 4)
    hipLaunchKernelGGL(k_build_narrow<4>, dim3(nb), dim3(64), 0, s, prm);
  else
    hipLaunchKernelGGL(k_build, dim3(nb), dim3(64), 0, s, prm);
  return hipGetLastError();
}
