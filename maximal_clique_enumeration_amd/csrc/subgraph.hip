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
// every P member after the rows, see mce_micro_table_words): header (p | x << 32), root id
// and |R| at the root, R's hash terms summed, rows (row a = bit b set iff L[a] ~ P[b], local order = id
// order, P first), p hash terms of the P members, p + x int32 ids.
//
// Two builds:
//  - micro tables (|P|, |X| <= 64): one 64-lane wavefront per root, one lane per
//    row;
//  - every other table, the split build: a head kernel writes each root's
//    header, ids and hash terms, then every root's rows, in slabs of 64, are
//    dealt over several blocks, so that one root with tens of thousands of rows
//    (X members of a hub in the full subgraph) is built by the whole chip.
// A row is filled either by walking the member's CSR row and looking every
// neighbour up in an LDS hash of P, or, for members of high degree, by probing
// each P member in that CSR row.
#include "mce_device.h"
#include "mce_internal.h"

// ------------------------------------------------------------------ a root's neighbourhood
// First-level root r (R = {r}): N(r), split at r. Second-level root, the CSR
// entry (v_i, v_j) with v_j the later end (R = {v_i, v_j}; section 3.2,
// Algorithm 4): N(v_i) n N(v_j), split at v_j, found by scanning the shorter of
// the two rows and searching the other. Either way the members come in id order.
struct RootHood {
  int sa, sb;      // the row scanned
  int oa, ob;      // the row searched for membership (oa < 0: none)
  const u64* hb;   // that row's owner's adjacency bitmap if it is a hub, else NULL
  int piv, pivr;   // P = the members after piv (round pivr), X = the others
  int k0;          // |R|
  u64 term;        // R's hash terms summed
};

// Adjacency bitmap of vertex v if it is a hub (second-level runs), else NULL:
// a membership test in its row is then one load instead of a binary search.
__device__ __forceinline__ const u64* hub_bitmap(const BuildParams& prm, int v) {
  if (!prm.hub_id) return nullptr;
  const int h = prm.hub_id[v];
  return h < 0 ? nullptr : prm.hub_bm + (size_t)h * prm.hub_words;
}

__device__ __forceinline__ RootHood root_hood(const BuildParams& prm, int rid) {
  const int* __restrict__ rp = prm.rp;
  RootHood h;
  if (!prm.l2) {
    h.sa = rp[rid];
    h.sb = rp[rid + 1];
    h.oa = h.ob = -1;
    h.hb = nullptr;
    h.piv = rid;
    h.pivr = prm.rnd[rid];
    h.k0 = 1;
    h.term = mce_vertex_term(rid);
  } else {
    const int vi = prm.src[rid], vj = prm.ci[rid];
    const int ai = rp[vi], bi = rp[vi + 1], aj = rp[vj], bj = rp[vj + 1];
    const bool si = bi - ai <= bj - aj;
    h.sa = si ? ai : aj;
    h.sb = si ? bi : bj;
    h.oa = si ? aj : ai;
    h.ob = si ? bj : bi;
    h.hb = hub_bitmap(prm, si ? vj : vi);
    h.piv = vj;
    h.pivr = prm.rnd[vj];
    h.k0 = 2;
    h.term = mce_vertex_term(vi) + mce_vertex_term(vj);
  }
  return h;
}

__device__ __forceinline__ bool hood_has(const int* __restrict__ ci, const RootHood& h, int u) {
  if (h.oa < 0) return true;
  if (h.hb) return (h.hb[u >> 6] >> (u & 63)) & 1ull;
  return csr_range_has(ci, h.oa, h.ob, u);
}

// ------------------------------------------------------------------ hash of P
// LDS open-addressing hash (key = vertex id, value = local index) over P.
template <int HB>
__device__ __forceinline__ u32 build_hash(int u) {
  return ((u32)u * 0x9E3779B1u) >> (32 - HB);
}

// Four binary searches for `key` in the sorted ranges [lo[z], hi[z]) of ci, in
// lockstep: the four loads of a step are independent and overlap.
__device__ __forceinline__ void csr_range_has4(const int* __restrict__ ci, const int lo_[4], const int hi_[4],
                                               int key, bool found[4]) {
  int lo[4], len[4];
#pragma unroll
  for (int z = 0; z < 4; z++) {
    lo[z] = lo_[z];
    len[z] = hi_[z] - lo_[z];
  }
  for (;;) {
    bool any = false;
    int v[4];
#pragma unroll
    for (int z = 0; z < 4; z++) v[z] = len[z] > 0 ? ci[lo[z] + (len[z] >> 1)] : 0;
#pragma unroll
    for (int z = 0; z < 4; z++) {
      if (len[z] > 0) {
        any = true;
        const int half = len[z] >> 1;
        if (v[z] < key) {
          lo[z] += half + 1;
          len[z] -= half + 1;
        } else {
          len[z] = half;
        }
      }
    }
    if (!any) break;
  }
#pragma unroll
  for (int z = 0; z < 4; z++) found[z] = lo[z] < hi_[z] && ci[lo[z]] == key;
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

// ------------------------------------------------------------------ micro tables
// |P| <= 64 and |X| <= 64: one wavefront per root, and the whole table (at most
// 128 one-word rows) is built in LDS. One pass over the root's CSR row splits it
// into P and X. Then, with the forward adjacency (prm.fadj): the ids of P u X go
// into an LDS hash, and the members' forward rows are streamed as one sequence,
// 64 consecutive entries per load (coalesced within a row), each entry's row
// found from the rows' length prefix sums; an edge between two members, found
// in the forward row of its earlier end, sets its bit in the row of each end
// that has a row over P (every row is over P, so: the X end's row if the other
// end is in P, and both rows if both are). Without it: P's ids go into the
// hash, the members' whole CSR rows are streamed the same way, and rows longer
// than 4 |P| are built by probing each P member in them. The X column of every
// P member (the transpose of the X rows) is taken in LDS, and the table is
// written out with coalesced stores.
#define MICRO_PROBE_RATIO 4   // rows longer than 4 |P| are probed
#define MICRO_MASK_CHUNKS 128 // forward-row slabs of up to 128 x 64 entries find rows by masks

__global__ __launch_bounds__(64) void k_build_micro(BuildParams prm) {
  constexpr int HB = 8;   // hash slots >= 2 * 128
  __shared__ int s_id[2 * MCE_MICRO_MAX];   // P ids, then X ids
  __shared__ int s_hk[1 << HB];
  __shared__ short s_hv[1 << HB];
  __shared__ int s_pre[MCE_WAVE];
  __shared__ int s_ga[MCE_WAVE];
  __shared__ u64 s_row[2 * MCE_MICRO_MAX];
  __shared__ u64 s_mask[MICRO_MASK_CHUNKS];   // per chunk of 64 streamed entries: bit j, a row starts at entry j
  __shared__ int s_nzr[MCE_WAVE];             // the slab's non-empty rows, in order
  const int lane = lane_id();
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ ci = prm.ci;
  const int* __restrict__ rnd = prm.rnd;
  for (int i = blockIdx.x; i < prm.nroots; i += gridDim.x) {
    const int r = prm.roots[i];
    const RootHood hd = root_hood(prm, r);
    const int a = hd.sa, b = hd.sb;
    // P (members after the root) and X (the others), each in id order
    int np = 0, nx = 0;
    for (int base = a; base < b; base += MCE_WAVE) {
      const int e = base + lane;
      const int u = e < b ? ci[e] : 0;
      const bool valid = e < b && hood_has(ci, hd, u);
      const bool lat = valid && order_after(rnd[u], u, hd.pivr, hd.piv);
      const u64 lm = ballot(lat), xm = ballot(valid && !lat);
      if (lat && np + mbcnt(lm) < MCE_MICRO_MAX) s_id[np + mbcnt(lm)] = u;
      if (valid && !lat && nx + mbcnt(xm) < MCE_MICRO_MAX) s_id[MCE_MICRO_MAX + nx + mbcnt(xm)] = u;
      np += __popcll(lm);
      nx += __popcll(xm);
    }
    if (np == 0 || np > MCE_MICRO_MAX || nx > MCE_MICRO_MAX) {   // the host sends only such roots here
      if (lane == 0) atomicOr(prm.status, MCE_E_LIMIT);
      continue;
    }
    const int nrows = np + nx;
    const u64 off = uni(prm.tab_off[i]) - uni(prm.tab_off[0]);
    if (off + mce_micro_table_words(np, nx) > prm.heap_words) {
      if (lane == 0) atomicOr(prm.status, MCE_E_HEAP);
      continue;
    }
    u64* T = prm.heap + off;
    u64* rows = T + 3;
    u64* xcol = rows + nrows;
    u64* hvs = xcol + np;
    int* ids = (int*)(hvs + np);
    if (lane == 0) {
      T[0] = (u64)(u32)np | ((u64)(u32)nx << 32);
      T[1] = (u64)(u32)r | ((u64)(u32)hd.k0 << 32);   // root id, |R| at the root
      T[2] = hd.term;
    }
    for (int h = lane; h < (1 << HB); h += MCE_WAVE) s_hk[h] = -1;
    __syncthreads();   // the ids are in LDS, the hash is clear
    const bool fwd = prm.fadj != nullptr;
    if (lane < np) {
      const int u = s_id[lane];
      ids[lane] = u;
      hvs[lane] = mce_vertex_term(u);
      u32 h = build_hash<HB>(u);
      while (atomicCAS(&s_hk[h], -1, u) != -1) h = (h + 1u) & ((1u << HB) - 1u);
      s_hv[h] = (short)lane;
    }
    if (lane < nx) {
      const int u = s_id[MCE_MICRO_MAX + lane];
      ids[np + lane] = u;
      if (fwd) {
        u32 h = build_hash<HB>(u);
        while (atomicCAS(&s_hk[h], -1, u) != -1) h = (h + 1u) & ((1u << HB) - 1u);
        s_hv[h] = (short)(np + lane);
      }
    }
    if (fwd) {
      for (int t = lane; t < nrows; t += MCE_WAVE) s_row[t] = 0;
      // forward rows, in slabs of 64 members (P members first, then X members)
      for (int t0 = 0; t0 < nrows; t0 += MCE_WAVE) {
        const int t = t0 + lane;
        int ga = 0, d = 0;
        if (t < nrows) {
          const int g = t < np ? s_id[t] : s_id[MCE_MICRO_MAX + t - np];
          ga = rp[g];
          d = prm.fdeg[g];
        }
        int inc = d;
#pragma unroll
        for (int o = 1; o < MCE_WAVE; o <<= 1) {
          const int v = __shfl_up(inc, o);
          if (lane >= o) inc += v;
        }
        const int D = uni(__shfl(inc, MCE_WAVE - 1));
        s_pre[lane] = inc - d;
        s_ga[lane] = ga;
        // Up to MICRO_MASK_CHUNKS chunks of 64 entries, an entry's row is found
        // from the chunk's mask of row starts: the non-empty rows in order, the
        // rows started at or before the entry in its chunk counted with one
        // popcount, plus those started before the chunk; else by a binary search
        // over the rows' prefix sums.
        const bool masks = D <= MICRO_MASK_CHUNKS * MCE_WAVE;
        if (masks) {
          for (int c = lane; c < (D + MCE_WAVE - 1) / MCE_WAVE; c += MCE_WAVE) s_mask[c] = 0;
          const u64 nz = ballot(d > 0);
          if (d > 0) s_nzr[mbcnt(nz)] = lane;
        }
        __syncthreads();   // the hash and cleared rows (first slab), the prefix sums, the cleared masks
        if (masks) {
          if (d > 0) atomicOr(&s_mask[(inc - d) >> 6], 1ull << ((inc - d) & 63));
          __syncthreads();
        }
        int started = 0;   // non-empty rows started before the current chunk
        for (int base = 0; base < D; base += 4 * MCE_WAVE) {
          int u[4], rw[4];
#pragma unroll
          for (int z = 0; z < 4; z++) {
            const int x = base + z * MCE_WAVE + lane;
            rw[z] = -1;
            u[z] = 0;
            int q = 0;   // the last row whose prefix is <= x
            if (masks) {
              const u64 m = base + z * MCE_WAVE < D ? s_mask[(base >> 6) + z] : 0ull;
              const u64 upto = lane == MCE_WAVE - 1 ? ~0ull : (2ull << lane) - 1ull;
              const int k = started + (int)__popcll(m & upto) - 1;   // >= 0 for every x < D
              q = s_nzr[k < 0 ? 0 : k];
              started += (int)__popcll(m);
            } else if (x < D) {
#pragma unroll
              for (int step = MCE_WAVE / 2; step > 0; step >>= 1)
                if (s_pre[q + step] <= x) q += step;
            }
            if (x < D) {
              rw[z] = q;
              u[z] = prm.fadj[s_ga[q] + (x - s_pre[q])];
            }
          }
#pragma unroll
          for (int z = 0; z < 4; z++) {
            if (rw[z] >= 0) {
              const int j = build_lookup<HB>(s_hk, s_hv, u[z]);
              const int ta = t0 + rw[z];
              if (j >= 0 && j < np) atomicOr(&s_row[ta], 1ull << j);
              if (j >= 0 && ta < np) atomicOr(&s_row[j], 1ull << ta);
            }
          }
        }
        __syncthreads();   // the prefix sums are rewritten by the next slab
      }
    }
    // rows, in slabs of 64 members (P members first, then X members)
    for (int t0 = 0; !fwd && t0 < nrows; t0 += MCE_WAVE) {
      const int t = t0 + lane;
      const bool valid = t < nrows;
      int ga = 0, d = 0, gv = 0;
      if (valid) {
        const int g = t < np ? s_id[t] : s_id[MCE_MICRO_MAX + t - np];
        gv = g;
        ga = rp[g];
        d = rp[g + 1] - ga;
      }
      const bool probe = valid && d > MICRO_PROBE_RATIO * np;
      const int dd = valid && !probe ? d : 0;
      int inc = dd;
#pragma unroll
      for (int o = 1; o < MCE_WAVE; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
      }
      const int D = uni(__shfl(inc, MCE_WAVE - 1));
      s_pre[lane] = inc - dd;
      s_ga[lane] = ga;
      s_row[t0 + lane] = 0;
      __syncthreads();   // the hash (first slab), the prefix sums and the cleared rows
      for (int base = 0; base < D; base += 4 * MCE_WAVE) {
        int u[4], rw[4];
#pragma unroll
        for (int z = 0; z < 4; z++) {
          const int x = base + z * MCE_WAVE + lane;
          rw[z] = -1;
          u[z] = 0;
          if (x < D) {
            int q = 0;   // the last row whose prefix is <= x
#pragma unroll
            for (int step = MCE_WAVE / 2; step > 0; step >>= 1)
              if (s_pre[q + step] <= x) q += step;
            rw[z] = q;
            u[z] = ci[s_ga[q] + (x - s_pre[q])];
          }
        }
#pragma unroll
        for (int z = 0; z < 4; z++) {
          if (rw[z] >= 0) {
            const int j = build_lookup<HB>(s_hk, s_hv, u[z]);
            if (j >= 0) atomicOr(&s_row[t0 + rw[z]], 1ull << j);
          }
        }
      }
      // rows much longer than P: probe each P member, several rows per pass when |P| is small
      const u64 pm = ballot(probe);
      if (pm) {
        const int npw = np <= 1 ? 1 : (np >= 64 ? 64 : 1 << (32 - __builtin_clz((u32)(np - 1))));
        const int per = MCE_WAVE / npw;   // rows per pass
        const int grp = lane / npw, jj = lane % npw;
        const int cntp = __popcll(pm);
        for (int c0 = 0; c0 < cntp; c0 += per) {
          int l = -1;   // the lane (row) of the (c0 + grp)-th probe row
          if (c0 + grp < cntp) {
            u64 m = pm;
            for (int q = 0; q < c0 + grp; q++) m &= m - 1ull;
            l = __builtin_ctzll(m);
          }
          const int gal = __shfl(ga, l < 0 ? 0 : l);
          const int gdl = __shfl(d, l < 0 ? 0 : l);
          const int gvl = __shfl(gv, l < 0 ? 0 : l);
          const u64* hb = l >= 0 ? hub_bitmap(prm, gvl) : nullptr;   // a hub row: one bit per probe
          const int key = jj < np ? s_id[jj] : 0;
          const bool found = l >= 0 && jj < np &&
                             (hb ? ((hb[key >> 6] >> (key & 63)) & 1ull) != 0ull : csr_range_has(ci, gal, gal + gdl, key));
          const u64 fm = ballot(found);
          if (jj == 0 && l >= 0) {
            const u64 mask = npw >= 64 ? ~0ull : ((1ull << npw) - 1ull);
            s_row[t0 + l] = (fm >> (grp * npw)) & mask;
          }
        }
      }
      __syncthreads();   // the slab's rows are complete
    }
    // X column of every P member (the X rows' bit of that member), then the rows
    if (lane < np) {
      u64 col = 0;
      for (int x2 = 0; x2 < nx; x2++) col |= ((s_row[np + x2] >> lane) & 1ull) << x2;
      xcol[lane] = col;
    }
    for (int t = lane; t < nrows; t += MCE_WAVE) rows[t] = s_row[t];
    __syncthreads();   // LDS is reused by the next root
  }
}

// ------------------------------------------------------------------ split build
// Head: one 256-thread block per root. The four wavefronts each take a quarter
// of the root's CSR row; a first pass counts its P (later) and X (earlier)
// members, a second writes them at their place in the table's id array.
__global__ __launch_bounds__(256) void k_build_head(BuildParams prm) {
  __shared__ int s_cnt[2][4];
  const int lane = lane_id();
  const int wv = (int)threadIdx.x >> 6;
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ ci = prm.ci;
  const int* __restrict__ rnd = prm.rnd;
  for (int i = blockIdx.x; i < prm.nroots; i += gridDim.x) {
    const int r = prm.roots[i];
    const RootHood hd = root_hood(prm, r);
    const int a = hd.sa, b = hd.sb;
    const int per = ((b - a + 4 * MCE_WAVE - 1) / (4 * MCE_WAVE)) * MCE_WAVE;
    const int wa = min(b, a + wv * per), wb = min(b, wa + per);
    int np = 0, nx = 0;
    for (int base = wa; base < wb; base += MCE_WAVE) {
      const int e = base + lane;
      const int u = e < wb ? ci[e] : 0;
      const bool valid = e < wb && hood_has(ci, hd, u);
      const bool lat = valid && order_after(rnd[u], u, hd.pivr, hd.piv);
      np += __popcll(ballot(lat));
      nx += __popcll(ballot(valid && !lat));
    }
    if (lane == 0) {
      s_cnt[0][wv] = np;
      s_cnt[1][wv] = nx;
    }
    __syncthreads();
    int NP = 0, NX = 0, pp = 0, xp = 0;
    for (int q = 0; q < 4; q++) {
      if (q == wv) {
        pp = NP;
        xp = NX;
      }
      NP += s_cnt[0][q];
      NX += s_cnt[1][q];
    }
    __syncthreads();   // s_cnt is read before the next root writes it
    const u64 off = uni(prm.tab_off[i]) - uni(prm.tab_off[0]);
    const u64 words = mce_table_words(NP, NX, prm.W, prm.mode);
    const bool fits = NP >= 1 && NP <= 64 * prm.W;   // the host sends only such roots here
    if (!fits || off + words > prm.heap_words) {
      // header with p = 0: the rows kernel skips the root
      if (threadIdx.x == 0) {
        if (off + 3 <= prm.heap_words) prm.heap[off] = 0;
        atomicOr(prm.status, fits ? MCE_E_HEAP : MCE_E_LIMIT);
      }
      continue;
    }
    u64* T = prm.heap + off;
    const long long nrows = mce_table_rows(NP, NX, prm.mode);
    u64* hvs = T + 3 + (size_t)nrows * prm.W;
    int* ids = (int*)(hvs + NP);
    if (threadIdx.x == 0) {
      T[0] = (u64)(u32)NP | ((u64)(u32)NX << 32);
      T[1] = (u64)(u32)r | ((u64)(u32)hd.k0 << 32);   // root id, |R| at the root
      T[2] = hd.term;
    }
    for (int base = wa; base < wb; base += MCE_WAVE) {
      const int e = base + lane;
      const int u = e < wb ? ci[e] : 0;
      const bool valid = e < wb && hood_has(ci, hd, u);
      const bool lat = valid && order_after(rnd[u], u, hd.pivr, hd.piv);
      const u64 lm = ballot(lat), xm = ballot(valid && !lat);
      if (lat) {
        const int j = pp + mbcnt(lm);
        ids[j] = u;
        hvs[j] = mce_vertex_term(u);
      } else if (valid) {
        ids[NP + xp + mbcnt(xm)] = u;
      }
      pp += __popcll(lm);
      xp += __popcll(xm);
    }
  }
}

// Rows: block (root i, part k) builds the slabs k, k + K, k + 2K, ... of root
// i's table. P's ids are read back from the table into an LDS hash (id -> local
// index). A slab's 64 CSR rows are streamed as one sequence: the wavefront reads
// 64 consecutive entries at a time (coalesced within each CSR row), finds each
// entry's row from the rows' degree prefix sums, and ORs the P members it finds
// into the slab's rows in LDS. The slab's work is then set by its total degree,
// not by its longest row. A row much longer than P is built instead by probing
// every P member in it. With the forward adjacency (prm.fadj), an X member's row
// is its forward row: every P member comes after every X member in the peel
// order (P after the pivot vertex, X before it), so the P members adjacent to
// it are all in that row, which is no longer than the member's core number.
// With the forward adjacency and W <= PROWS_MAX_W, the P rows are built by
// k_build_prows instead, and this kernel's slabs cover the X rows only.
#define SPLIT_STREAM_RATIO 2
#define PROWS_MAX_W 8

template <int W>
__host__ __device__ constexpr int build_hash_bits() {   // 2^HB >= 2 PMAX
  return W == 1 ? 7 : W == 2 ? 8 : W == 4 ? 9 : W == 8 ? 10 : W == 16 ? 11 : 12;
}

template <int W>
__global__ __launch_bounds__(64) void k_build_rows(BuildParams prm) {
  constexpr int PMAX = 64 * W;
  constexpr int HB = build_hash_bits<W>();
  __shared__ int s_hk[1 << HB];
  __shared__ short s_hv[1 << HB];
  __shared__ int s_pre[MCE_WAVE];   // exclusive prefix sum of the slab rows' streamed degrees
  __shared__ int s_ga[MCE_WAVE];    // their CSR row starts
  __shared__ int s_fw[MCE_WAVE];    // 1: the row streamed is the forward row
  __shared__ u64 s_slab[MCE_WAVE * W];
  const int lane = lane_id();
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ ci = prm.ci;
  const int mode = prm.mode;
  const int K = prm.parts;
  const long long items = (long long)prm.nroots * K;
  int cur = -1;   // the root whose P is in LDS
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int i = (int)(it / K), k = (int)(it % K);
    const u64 off = uni(prm.tab_off[i]) - uni(prm.tab_off[0]);
    if (off + 3 > prm.heap_words) continue;
    u64* T = prm.heap + off;
    const u64 hdr = uni(T[0]);
    const int np = (int)(u32)hdr, nx = (int)(u32)(hdr >> 32);
    if (np < 1 || np > PMAX) continue;   // the head kernel flagged this root
    const int nrows = (int)mce_table_rows(np, nx, mode);
    const int rfirst = prm.fadj && W <= PROWS_MAX_W ? np : 0;   // the first row built here
    const int nslab = (nrows - rfirst + MCE_WAVE - 1) / MCE_WAVE;
    if (k >= nslab) continue;
    if (off + mce_table_words(np, nx, W, mode) > prm.heap_words) continue;
    u64* rows = T + 3;
    const u64* hvs = rows + (size_t)nrows * W;
    const int* ids = (const int*)(hvs + np);
    if (i != cur) {
      __syncthreads();   // the previous root's hash is no longer read
      for (int h = lane; h < (1 << HB); h += MCE_WAVE) s_hk[h] = -1;
      __syncthreads();
      for (int j = lane; j < np; j += MCE_WAVE) {
        const int u = ids[j];
        u32 h = build_hash<HB>(u);
        while (atomicCAS(&s_hk[h], -1, u) != -1) h = (h + 1u) & ((1u << HB) - 1u);
        s_hv[h] = (short)j;
      }
      __syncthreads();
      cur = i;
    }
    for (int slab = k; slab < nslab; slab += K) {
      const int t0 = rfirst + slab * MCE_WAVE;
      const int t = t0 + lane;
      const bool valid = t < nrows;
      int ga = 0, d = 0, gv = 0;
      const bool fw = valid && prm.fadj && t >= np;   // an X member's row, from its forward row
      if (valid) {
        const int g = ids[t];
        gv = g;
        ga = rp[g];
        d = fw ? prm.fdeg[g] : rp[g + 1] - ga;
      }
      const bool probe = valid && !fw && d > SPLIT_STREAM_RATIO * np;
      const int dd = valid && !probe ? d : 0;
      int inc = dd;
#pragma unroll
      for (int o = 1; o < MCE_WAVE; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
      }
      const int D = uni(__shfl(inc, MCE_WAVE - 1));
      s_pre[lane] = inc - dd;
      s_ga[lane] = ga;
      s_fw[lane] = fw ? 1 : 0;
      for (int q = lane; q < MCE_WAVE * W; q += MCE_WAVE) s_slab[q] = 0;
      __syncthreads();
      for (int base = 0; base < D; base += 4 * MCE_WAVE) {
        int u[4], rr[4];
#pragma unroll
        for (int z = 0; z < 4; z++) {
          const int x = base + z * MCE_WAVE + lane;
          rr[z] = -1;
          u[z] = -1;
          if (x < D) {
            int r = 0;   // the last row whose prefix is <= x (it has x - prefix < its degree)
#pragma unroll
            for (int step = MCE_WAVE / 2; step > 0; step >>= 1)
              if (s_pre[r + step] <= x) r += step;
            rr[z] = r;
            u[z] = (s_fw[r] ? prm.fadj : ci)[s_ga[r] + (x - s_pre[r])];
          }
        }
#pragma unroll
        for (int z = 0; z < 4; z++) {
          if (rr[z] >= 0) {
            const int j = build_lookup<HB>(s_hk, s_hv, u[z]);
            if (j >= 0) atomicOr(&s_slab[rr[z] * W + (j >> 6)], 1ull << (j & 63));
          }
        }
      }
      __syncthreads();
      const u64 pm = ballot(probe);
      const int nr = min(MCE_WAVE, nrows - t0);
      u64* srow = rows + (size_t)t0 * W;
      for (int q = lane; q < nr * W; q += MCE_WAVE)
        if (!((pm >> (q / W)) & 1ull)) srow[q] = s_slab[q];
      // rows much longer than P: probe every P member in the CSR row, four rows
      // at a time (their binary searches run in lockstep, so the loads overlap)
      for (u64 m = pm; m != 0;) {
        int lr[4], lo[4], hi[4];
        const u64* hbz[4];   // a hub's row: bit tests instead of the search
#pragma unroll
        for (int z = 0; z < 4; z++) {
          lr[z] = m ? __builtin_ctzll(m) : -1;
          m = m ? (m & (m - 1ull)) : 0ull;
          hbz[z] = lr[z] >= 0 ? hub_bitmap(prm, read_lane(gv, lr[z])) : nullptr;
          lo[z] = lr[z] >= 0 ? read_lane(ga, lr[z]) : 0;
          hi[z] = lr[z] >= 0 && !hbz[z] ? lo[z] + read_lane(d, lr[z]) : lo[z];
        }
        for (int w0 = 0; w0 < W; w0++) {
          const int j = w0 * 64 + lane;
          const int key = j < np ? ids[j] : -1;
          bool f[4];
          csr_range_has4(ci, lo, hi, key, f);
#pragma unroll
          for (int z = 0; z < 4; z++)
            if (hbz[z]) f[z] = key >= 0 && ((hbz[z][key >> 6] >> (key & 63)) & 1ull) != 0ull;
#pragma unroll
          for (int z = 0; z < 4; z++) {
            const u64 fm = ballot(f[z] && j < np);
            if (lane == 0 && lr[z] >= 0) srow[(size_t)lr[z] * W + w0] = fm;
          }
        }
      }
      __syncthreads();   // s_pre, s_ga and s_slab are rewritten by the next slab
    }
  }
}

// P rows from the forward adjacency: block i builds every P row of root i in
// LDS. The forward rows of the P members are streamed, 64 members (a slab) at a
// time as one sequence, its entries dealt over the block's four wavefronts 64 at
// a time with four loads in flight per lane, each entry's member found from the
// slab's prefix sums of forward degrees. An entry that is a P member is an edge
// between two P members, seen from its earlier end in the peel order, and it
// sets its bit in the rows of both ends; every such edge lies in exactly one of
// the forward rows streamed, so each row is complete once all are. A forward
// row is no longer than the member's core number, where the CSR rows of P's hub
// members run to thousands of entries (each P member was looked up in them by
// binary search).
template <int W>
__global__ __launch_bounds__(256) void k_build_prows(BuildParams prm) {
  constexpr int PMAX = 64 * W;
  constexpr int HB = build_hash_bits<W>();
  constexpr int NWV = 4;   // wavefronts per block
  __shared__ int s_hk[1 << HB];
  __shared__ short s_hv[1 << HB];
  __shared__ int s_pre[MCE_WAVE];   // exclusive prefix sum of the slab members' forward degrees
  __shared__ int s_ga[MCE_WAVE];    // their row starts
  __shared__ int s_D;               // the slab's total
  __shared__ u64 s_rows[PMAX * W];
  const int lane = lane_id();
  const int wv = (int)threadIdx.x / MCE_WAVE;
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ fadj = prm.fadj;
  const int* __restrict__ fdeg = prm.fdeg;
  for (int i = blockIdx.x; i < prm.nroots; i += gridDim.x) {
    const u64 off = uni(prm.tab_off[i]) - uni(prm.tab_off[0]);
    if (off + 3 > prm.heap_words) continue;
    u64* T = prm.heap + off;
    const u64 hdr = uni(T[0]);
    const int np = (int)(u32)hdr, nx = (int)(u32)(hdr >> 32);
    if (np < 1 || np > PMAX) continue;   // the head kernel flagged this root
    const int nrows = (int)mce_table_rows(np, nx, prm.mode);
    if (off + mce_table_words(np, nx, W, prm.mode) > prm.heap_words) continue;
    u64* rows = T + 3;
    const u64* hvs = rows + (size_t)nrows * W;
    const int* ids = (const int*)(hvs + np);
    __syncthreads();   // the previous root's rows are written out, its hash no longer read
    for (int h = threadIdx.x; h < (1 << HB); h += blockDim.x) s_hk[h] = -1;
    for (int q = threadIdx.x; q < np * W; q += blockDim.x) s_rows[q] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < np; j += blockDim.x) {
      const int u = ids[j];
      u32 h = build_hash<HB>(u);
      while (atomicCAS(&s_hk[h], -1, u) != -1) h = (h + 1u) & ((1u << HB) - 1u);
      s_hv[h] = (short)j;
    }
    for (int t0 = 0; t0 < np; t0 += MCE_WAVE) {
      if (wv == 0) {
        const int t = t0 + lane;
        int ga = 0, d = 0;
        if (t < np) {
          const int g = ids[t];
          ga = rp[g];
          d = fdeg[g];
        }
        int inc = d;
#pragma unroll
        for (int o = 1; o < MCE_WAVE; o <<= 1) {
          const int v = __shfl_up(inc, o);
          if (lane >= o) inc += v;
        }
        s_pre[lane] = inc - d;
        s_ga[lane] = ga;
        if (lane == MCE_WAVE - 1) s_D = inc;
      }
      __syncthreads();   // the hash (first slab) and the slab's prefix sums
      const int D = s_D;
      for (int base = wv * MCE_WAVE; base < D; base += 4 * NWV * MCE_WAVE) {
        int u[4], rr[4];
#pragma unroll
        for (int z = 0; z < 4; z++) {
          const int x = base + z * NWV * MCE_WAVE + lane;
          rr[z] = -1;
          u[z] = -1;
          if (x < D) {
            int r = 0;   // the last member whose prefix is <= x (it has x - prefix < its degree)
#pragma unroll
            for (int step = MCE_WAVE / 2; step > 0; step >>= 1)
              if (s_pre[r + step] <= x) r += step;
            rr[z] = r;
            u[z] = fadj[s_ga[r] + (x - s_pre[r])];
          }
        }
#pragma unroll
        for (int z = 0; z < 4; z++) {
          if (rr[z] >= 0) {
            const int j = build_lookup<HB>(s_hk, s_hv, u[z]);
            if (j >= 0) {
              const int a = t0 + rr[z];
              atomicOr(&s_rows[a * W + (j >> 6)], 1ull << (j & 63));
              atomicOr(&s_rows[j * W + (a >> 6)], 1ull << (a & 63));
            }
          }
        }
      }
      __syncthreads();   // the slab's prefix sums are rewritten by the next slab; the rows are complete
    }
    for (int q = threadIdx.x; q < np * W; q += blockDim.x) rows[q] = s_rows[q];
  }
}

hipError_t mce_launch_build(const BuildParams& prm, int blocks, hipStream_t s) {
  if (prm.micro) {
    const int nb = std::max(1, std::min(blocks, prm.nroots));
    hipLaunchKernelGGL(k_build_micro, dim3(nb), dim3(64), 0, s, prm);
    return hipGetLastError();
  }
  if (prm.parts < 1) return hipErrorInvalidValue;
  const int nh = std::max(1, std::min(blocks / 4, prm.nroots));
  hipLaunchKernelGGL(k_build_head, dim3(nh), dim3(256), 0, s, prm);
  if (prm.fadj && prm.W <= PROWS_MAX_W) {
    const int np = std::max(1, std::min(blocks / 4, prm.nroots));
    switch (prm.W) {
      case 1: hipLaunchKernelGGL(k_build_prows<1>, dim3(np), dim3(256), 0, s, prm); break;
      case 2: hipLaunchKernelGGL(k_build_prows<2>, dim3(np), dim3(256), 0, s, prm); break;
      case 4: hipLaunchKernelGGL(k_build_prows<4>, dim3(np), dim3(256), 0, s, prm); break;
      case 8: hipLaunchKernelGGL(k_build_prows<8>, dim3(np), dim3(256), 0, s, prm); break;
      default: return hipErrorInvalidValue;
    }
  }
  const long long items = (long long)prm.nroots * prm.parts;
  const int nb = (int)std::max(1LL, std::min((long long)blocks, items));
  switch (prm.W) {
    case 1: hipLaunchKernelGGL(k_build_rows<1>, dim3(nb), dim3(64), 0, s, prm); break;
    case 2: hipLaunchKernelGGL(k_build_rows<2>, dim3(nb), dim3(64), 0, s, prm); break;
    case 4: hipLaunchKernelGGL(k_build_rows<4>, dim3(nb), dim3(64), 0, s, prm); break;
    case 8: hipLaunchKernelGGL(k_build_rows<8>, dim3(nb), dim3(64), 0, s, prm); break;
    case 16: hipLaunchKernelGGL(k_build_rows<16>, dim3(nb), dim3(64), 0, s, prm); break;
    case 32: hipLaunchKernelGGL(k_build_rows<32>, dim3(nb), dim3(64), 0, s, prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
