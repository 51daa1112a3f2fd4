// Preprocessing before the search: input checks, the degeneracy order and the
// split of every vertex's neighbourhood into later (P) and earlier (X) parts.
//
// "Parallelizing Maximal Clique Enumeration on GPUs" (arxiv 2212.01473v2):
//  - section 2.1: the input is a simple undirected graph;
//  - section 2.4 (degeneracy ordering): order the vertices so that each has at
//    most d later neighbours; section 4.1 counts this preprocessing as timed work;
//  - section 2.4, Algorithm 3: root v_i gets P = later neighbours, X = earlier.
#include "mce_device.h"
#include "mce_internal.h"

#include <algorithm>

// ------------------------------------------------------------------ validation
// Pass 1: row_ptr is monotone and inside [0, nnz]; degrees; Delta.
__global__ __launch_bounds__(256) void k_validate_rowptr(int n, long long nnz, const int* __restrict__ rp,
                                                          MceCtl* ctl) {
  u32 bad = 0;
  int dmax = 0;
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < n; v += gridDim.x * blockDim.x) {
    int a = rp[v], b = rp[v + 1];
    if (a > b || a < 0 || (long long)b > nnz) bad |= 1u;   // MCE_GRAPH_ROWPTR
    else dmax = max(dmax, b - a);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (rp[0] != 0 || (long long)rp[n] != nnz) bad |= 1u;
  }
  u32 b = wave_or_u32(bad);
  u32 m = wave_max_u32((u32)dmax);
  if (lane_id() == 0) {
    if (b) atomicOr(&ctl->status, b);
    if (m) atomicMax(&ctl->max_degree, (int)m);
  }
}

// Pass 2 (only if pass 1 found nothing): ids in range, no loops, rows strictly
// ascending, and every edge present in both directions. One wavefront per row.
__global__ __launch_bounds__(256) void k_validate_cols(int n, const int* __restrict__ rp,
                                                        const int* __restrict__ ci, MceCtl* ctl) {
  if (ld_relaxed(&ctl->status) != 0) return;
  const int lane = lane_id();
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / MCE_WAVE;
  const int nwaves = gridDim.x * blockDim.x / MCE_WAVE;
  u32 bad = 0;
  for (int v = wave; v < n; v += nwaves) {
    int a = rp[v], b = rp[v + 1];
    for (int e = a + lane; e < b; e += MCE_WAVE) {
      int u = ci[e];
      if (u < 0 || u >= n) {
        bad |= 2u;                                 // MCE_GRAPH_RANGE
        continue;
      }
      if (u == v) bad |= 4u;                       // MCE_GRAPH_LOOP
      if (e + 1 < b && ci[e + 1] <= u) bad |= 8u;  // MCE_GRAPH_ORDER
      if (!csr_range_has(ci, rp[u], rp[u + 1], v)) bad |= 16u;  // MCE_GRAPH_ASYM
    }
  }
  u32 bb = wave_or_u32(bad);
  if (lane == 0 && bb) atomicOr(&ctl->status, bb);
}

// ------------------------------------------------------------------ k-core peel
// Grid-wide barrier for a cooperative launch, without agent-scope fences (their
// L2 write-back / invalidate serialises when hundreds of blocks issue them).
// Everything the peel passes between blocks is read and written with
// agent-scope relaxed atomics, which are performed at the device coherence
// point; the barrier only has to order them: each block waits until its own
// memory operations completed, then arrives. The arrival counter only grows
// (it is zeroed with the control block before the launch): barrier number e of
// the launch is complete once it reaches e * gridDim.x, so no block has to
// reset it or open a generation, and a block needs one atomic add and its
// polls. Bounded: past the deadline it flags MCE_E_TIMEOUT and lets the block
// go; the caller checks the flag after every barrier.
__device__ void grid_sync(MceCtl* ctl, u64 deadline, u32& epoch, bool solo = false) {
  wait_stores_complete();
  __syncthreads();
  if (gridDim.x > 1 && !solo) {
    if (threadIdx.x == 0) {
      epoch++;
      const u32 target = epoch * gridDim.x;
      __hip_atomic_fetch_add(&ctl->bar_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      u32 spins = 0;
      while (ld_relaxed(&ctl->bar_count) < target) {
        __builtin_amdgcn_s_sleep(1);
        if ((++spins & 1023u) == 0 && past_deadline(deadline)) {
          atomicOr(&ctl->status, MCE_E_TIMEOUT);
          break;
        }
      }
    }
    __syncthreads();
  }
}

// Peel memory operations at a chosen scope: agent scope while the whole grid
// works (the blocks sit on different XCDs, whose L2s are not coherent with each
// other), workgroup scope once block 0 works alone (its XCD's L2 is then the
// only cache that matters, and an operation is an L2 round trip instead of one
// to the device coherence point).
#define SA __HIP_MEMORY_SCOPE_AGENT
#define SW __HIP_MEMORY_SCOPE_WORKGROUP
template <int S>
__device__ __forceinline__ int pld(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, S);
}
template <int S>
__device__ __forceinline__ void pst(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, S);
}
template <int S>
__device__ __forceinline__ int padd(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, S);
}
template <int S>
__device__ __forceinline__ void pmin(int* p, int v) {
  __hip_atomic_fetch_min(p, v, __ATOMIC_RELAXED, S);
}

// Vertices whose CSR row is longer than PEEL_BIG join the big frontier, whose
// rows are split into PEEL_SPAN-edge spans shared by all waves of the round.
#ifndef PEEL_BIG
#define PEEL_BIG 512
#endif
#define PEEL_SPAN (4 * MCE_WAVE)
#ifndef PEEL_SOLO
#define PEEL_SOLO 4096
#endif
#define PEEL_THREADS 1024

// Appends the lanes with `in` set to the next frontier: the regular list, or
// the big list for vertices of degree > PEEL_BIG. Whole wave.
template <int S>
__device__ __forceinline__ void peel_append(bool in, int v, const int* __restrict__ rp, int* fr, int* fsize,
                                            int* bfr, int* bsize) {
  const int lane = lane_id();
  const bool big = in && rp[v + 1] - rp[v] > PEEL_BIG;
  const u64 mr = ballot(in && !big);
  const u64 mb = ballot(big);
  int pr = 0, pb = 0;
  if (lane == 0 && mr) pr = padd<S>(fsize, __popcll(mr));
  if (lane == 0 && mb) pb = padd<S>(bsize, __popcll(mb));
  pr = read_lane(pr, 0);
  pb = read_lane(pb, 0);
  if (in && !big) pst<S>(&fr[pr + mbcnt(mr)], v);
  if (big) pst<S>(&bfr[pb + mbcnt(mb)], v);
}

// One span of a removed vertex's row [base, min(base + PEEL_SPAN, b)): take one
// degree from each neighbour (all four 64-edge pieces in flight together). A
// neighbour that falls from k + 1 to k joins the next round. The decrement is
// unconditional: a vertex already removed has degree <= k at its removal and
// only loses more, so it never falls from k + 1 again; its degree is not read.
template <int S>
__device__ __forceinline__ void peel_span(int base, int b, int k, const int* __restrict__ rp,
                                          const int* __restrict__ ci, int* deg, int* nx, int* nxs, int* bnx,
                                          int* bnxs) {
  const int lane = lane_id();
  int u[4];
  bool ok[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int e = base + q * MCE_WAVE + lane;
    ok[q] = e < b;
    u[q] = ok[q] ? ci[e] : 0;
  }
  bool joins[4];
#pragma unroll
  for (int q = 0; q < 4; q++) joins[q] = ok[q] && padd<S>(&deg[u[q]], -1) == k + 1;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if (ballot(joins[q])) peel_append<S>(joins[q], u[q], rp, nx, nxs, bnx, bnxs);
  }
}

struct PeelArgs {
  int n;
  const int* rp;
  const int* ci;
  int* deg;
  int* rnd;
  int* core;
  int* alive0;
  int* alive1;
  int* front0;
  int* front1;
  int* bfront0;
  int* bfront1;
  MceCtl* ctl;
  u64 deadline;
  // ping-pong buffers by parity (selects, not indexed arrays: no scratch memory)
  __device__ int* alive(int i) const { return (i & 1) ? alive1 : alive0; }
  __device__ int* front(int i) const { return (i & 1) ? front1 : front0; }
  __device__ int* bfront(int i) const { return (i & 1) ? bfront1 : bfront0; }
};

struct PeelState {
  int cur, nf, nb, k, r, na;
  bool level_known;     // the level's remaining list and k are known, its first round is not built
  u32 epoch;            // grid barriers passed (thread 0 of each block)
  u64 tb, tl, tr, tm;   // first block's thread 0: barrier, level, round ticks; last mark
};

#define PEEL_MARK(acc)                \
  if (timer) {                        \
    const u64 t = wall_clock64();     \
    st.acc += t - st.tm;              \
    st.tm = t;                        \
  }

// Rounds of the peel at scope S (see k_peel). `wave`/`nwaves` index the waves
// taking part. Returns 0 when every vertex is ordered, 1 when the remaining
// list has shrunk to PEEL_SOLO vertices or fewer (grid phase only), -1 on a
// time-out.
template <int S, bool SOLO>
__device__ int peel_rounds(const PeelArgs& A, PeelState& st, int wave, int nwaves, bool timer) {
  const int lane = lane_id();
  const bool lead = SOLO ? threadIdx.x == 0 : (blockIdx.x == 0 && threadIdx.x == 0);
  MceCtl* ctl = A.ctl;
  const int* rp = A.rp;
  for (;;) {
    if (st.nf == 0 && st.nb == 0) {
      if (!st.level_known) {
      // new level: compact the remaining list and find the smallest remaining degree
      const int* src = A.alive(st.cur);
      int* dst = A.alive(st.cur ^ 1);
      int mn = 0x7FFFFFFF;
      for (int base = wave * MCE_WAVE; base < st.na; base += nwaves * MCE_WAVE) {
        const int i = base + lane;
        bool keep = false;
        int v = 0;
        if (i < st.na) {
          v = pld<S>(&src[i]);
          keep = pld<S>(&A.rnd[v]) < 0;
          if (keep) mn = min(mn, pld<S>(&A.deg[v]));
        }
        const u64 m = ballot(keep);
        int pos = 0;
        if (lane == 0 && m) pos = padd<S>(&ctl->asize[st.cur ^ 1], __popcll(m));
        pos = read_lane(pos, 0);
        if (keep) pst<S>(&dst[pos + mbcnt(m)], v);
      }
      const int wmn = wave_min_i32_nonneg(mn);
      if (lane == 0 && wmn != 0x7FFFFFFF) pmin<S>(&ctl->min_deg, wmn);
      PEEL_MARK(tl);
      grid_sync(ctl, A.deadline, st.epoch, SOLO);
      PEEL_MARK(tb);
      st.cur ^= 1;
      const u32 status = ld_relaxed(&ctl->status);
      st.na = pld<S>(&ctl->asize[st.cur]);
      const int kmin = pld<S>(&ctl->min_deg);   // no remaining vertex: k stays the degeneracy
      if (status & MCE_E_TIMEOUT) return -1;
      if (st.na == 0) return 0;
      st.k = kmin;
      if (!SOLO && gridDim.x > 1 && st.na <= PEEL_SOLO) {
        st.level_known = true;
        return 1;
      }
      }
      st.level_known = false;
      // the level's first round: every remaining vertex of degree <= k
      const int* al = A.alive(st.cur);
      for (int base = wave * MCE_WAVE; base < st.na; base += nwaves * MCE_WAVE) {
        const int i = base + lane;
        bool in = false;
        int v = 0;
        if (i < st.na) {
          v = pld<S>(&al[i]);
          in = pld<S>(&A.deg[v]) <= st.k;
        }
        peel_append<S>(in, v, rp, A.front(st.r), &ctl->fsize[st.r % 3], A.bfront(st.r),
                       &ctl->bsize[st.r % 3]);
      }
      PEEL_MARK(tl);
      grid_sync(ctl, A.deadline, st.epoch, SOLO);
      PEEL_MARK(tb);
      const u32 status2 = ld_relaxed(&ctl->status);
      st.nf = pld<S>(&ctl->fsize[st.r % 3]);
      st.nb = pld<S>(&ctl->bsize[st.r % 3]);
      if (status2 & MCE_E_TIMEOUT) return -1;
    }
    // round r: remove the frontier, take one degree from each neighbour
    const int r = st.r, k = st.k;
    if (lead) {
      // counters nobody reads any more: the frontier sizes read two rounds ago,
      // the old remaining-list size and the level's minimum
      pst<S>(&ctl->fsize[(r + 2) % 3], 0);
      pst<S>(&ctl->bsize[(r + 2) % 3], 0);
      pst<S>(&ctl->asize[st.cur ^ 1], 0);
      pst<S>(&ctl->min_deg, 0x7FFFFFFF);
    }
    const int* fr = A.front(r);
    const int* bfr = A.bfront(r);
    int* nx = A.front(r + 1);
    int* nxs = &ctl->fsize[(r + 1) % 3];
    int* bnx = A.bfront(r + 1);
    int* bnxs = &ctl->bsize[(r + 1) % 3];
    // vertices of small degree: one wave each
    for (int i = wave; i < st.nf; i += nwaves) {
      const int v = pld<S>(&fr[i]);
      if (lane == 0) {
        pst<S>(&A.rnd[v], r);
        A.core[v] = k;
      }
      const int a = rp[v], b = rp[v + 1];
      for (int base = a; base < b; base += PEEL_SPAN) peel_span<S>(base, b, k, rp, A.ci, A.deg, nx, nxs, bnx, bnxs);
    }
    // vertices of large degree: their spans are dealt round-robin to all waves
    for (int j0 = 0; j0 < st.nb; j0 += MCE_WAVE) {
      const int jl = j0 + lane;
      const int vl = jl < st.nb ? pld<S>(&bfr[jl]) : 0;
      const int al = jl < st.nb ? rp[vl] : 0;
      const int bl = jl < st.nb ? rp[vl + 1] : 0;
      const int cnt = min(MCE_WAVE, st.nb - j0);
      for (int t = 0; t < cnt; t++) {
        const int j = j0 + t;
        const int v = read_lane(vl, t);
        const int a = read_lane(al, t);
        const int b = read_lane(bl, t);
        if (j % nwaves == wave && lane == 0) {
          pst<S>(&A.rnd[v], r);
          A.core[v] = k;
        }
        const int nsp = (b - a + PEEL_SPAN - 1) / PEEL_SPAN;
        for (int c = (wave - j % nwaves + nwaves) % nwaves; c < nsp; c += nwaves)
          peel_span<S>(a + c * PEEL_SPAN, b, k, rp, A.ci, A.deg, nx, nxs, bnx, bnxs);
      }
    }
    PEEL_MARK(tr);
    grid_sync(ctl, A.deadline, st.epoch, SOLO);
    PEEL_MARK(tb);
    const u32 status = ld_relaxed(&ctl->status);
    st.nf = pld<S>(nxs);
    st.nb = pld<S>(bnxs);
    st.r++;
    if (status & MCE_E_TIMEOUT) return -1;
  }
}

// Round-synchronous peel (section 2.4 asks for a degeneracy order; this is the
// one the engine uses). Level k: every remaining vertex of current degree <= k
// leaves in one round (rnd = round, core = k). The removed vertices'
// neighbours lose one degree each, and a neighbour whose degree falls from k+1
// to k joins the next round of the same level; when a round removes nothing, k
// becomes the smallest remaining degree. Marking the round's vertices and
// decrementing their neighbours happen in the same phase: a vertex of the
// current round already has degree <= k, so a decrement can never make it join
// again (that needs a fall from k+1). One grid barrier per round. Launched
// cooperatively; one block for small graphs. Late rounds are small (the
// remaining graph is the dense core), so once at most PEEL_SOLO vertices remain
// block 0 finishes alone at workgroup scope and the other blocks leave.
__global__ __launch_bounds__(PEEL_THREADS) void k_peel(int n, const int* __restrict__ rp,
                                                        const int* __restrict__ ci, int* deg, int* rnd, int* core,
                                                        int* alive0, int* alive1, int* front0, int* front1,
                                                        int* bfront0, int* bfront1, MceCtl* ctl, u64 budget) {
  if (ld_relaxed(&ctl->status) != 0) return;   // rejected input: nothing to order
  const u64 t0 = wall_clock64();
  PeelArgs A{n, rp, ci, deg, rnd, core, alive0, alive1, front0, front1, bfront0, bfront1, ctl, t0 + budget};
  const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
  const int gsize = gridDim.x * blockDim.x;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  PeelState st{0, 0, 0, 0, 0, n, false, 0u, 0, 0, 0, t0};

  for (int v = gtid; v < n; v += gsize) {
    pst<SA>(&deg[v], rp[v + 1] - rp[v]);
    pst<SA>(&rnd[v], -1);
    pst<SA>(&alive0[v], v);
  }
  if (gtid == 0) {
    st_relaxed64(&ctl->t_run, t0);
    pst<SA>(&ctl->asize[0], n);
    pst<SA>(&ctl->asize[1], 0);
    for (int i = 0; i < 3; i++) {
      pst<SA>(&ctl->fsize[i], 0);
      pst<SA>(&ctl->bsize[i], 0);
    }
    pst<SA>(&ctl->min_deg, 0x7FFFFFFF);
  }
  grid_sync(ctl, A.deadline, st.epoch);

  int res;
  if (gridDim.x > 1) {
    res = peel_rounds<SA, false>(A, st, gtid / MCE_WAVE, gsize / MCE_WAVE, timer);
    if (res == 1) {
      if (blockIdx.x != 0) return;
      // block 0 goes on alone: drop any stale copy its XCD's caches may hold
      // of what the other blocks wrote
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      res = peel_rounds<SW, true>(A, st, threadIdx.x / MCE_WAVE, blockDim.x / MCE_WAVE, timer);
    }
  } else {
    res = peel_rounds<SW, true>(A, st, threadIdx.x / MCE_WAVE, blockDim.x / MCE_WAVE, timer);
  }
  if (res < 0) return;
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    ctl->rounds = st.r;
    ctl->degeneracy = st.k;
    ctl->peel_ticks[0] = st.tb;
    ctl->peel_ticks[1] = st.tl;
    ctl->peel_ticks[2] = st.tr;
    ctl->peel_ticks[3] = wall_clock64() - t0;
  }
}
#undef PEEL_MARK


// ------------------------------------------------------------------ orientation
// Per root: |P| = later neighbours, |X| = earlier ones. Degree-0 roots are
// maximal cliques of size 1 and are counted here. Roots with 1 <= |P| <= MCE_MAX_P
// are tallied per sub-class under every classification variant (subgraph mode,
// micro sub-class on or off): count, largest |P|, |X| and row count, heap
// words, so that the host can pick the variant and size every launch from one
// read-back.
__global__ __launch_bounds__(256) void k_orient(int n, const int* __restrict__ rp, const int* __restrict__ ci,
                                                 const int* __restrict__ rnd, const int* __restrict__ roots,
                                                 int nroots, int* pcount, int* xcount, MceCtl* ctl) {
  if (ld_relaxed(&ctl->status) != 0) return;
  const int lane = lane_id();
  const int gsize = gridDim.x * blockDim.x;
  const int cnt = nroots;   // roots == NULL: the identity list 0..nroots-1
  u64 iso = 0, iso_hash = 0;
  int pmax = 0, xmax = 0, dmax = 0;
  u32 lim = 0;
  for (int base = blockIdx.x * blockDim.x; base < cnt; base += gsize) {
    const int i = base + threadIdx.x;
    int p = 0, x = 0;
    bool valid = false;
    const int v = i < cnt ? (roots ? roots[i] : i) : 0;
    if (i < cnt && (v < 0 || v >= n)) {   // caller-supplied root out of range: flag it, touch nothing
      lim |= 2u;
      pcount[i] = 0;
      xcount[i] = 0;
    } else if (i < cnt) {
      const int a = rp[v], b = rp[v + 1];
      const int rv = rnd[v];
      for (int e = a; e < b; e++) {
        const int u = ci[e];
        p += order_after(rnd[u], u, rv, v) ? 1 : 0;
      }
      x = (b - a) - p;
      pcount[i] = p;
      xcount[i] = x;
      if (b == a) {
        iso++;
        iso_hash += mce_clique_term(mce_vertex_term(v), 1);
      }
      pmax = max(pmax, p);
      xmax = max(xmax, x);
      dmax = max(dmax, b - a);
      if (p > MCE_MAX_P) lim |= 1u;
      valid = p > 0 && p <= MCE_MAX_P;
    }
    for (int var = 0; var < MCE_NVAR; var++) {
      const int mode = var & 1;
      const int sub = valid ? mce_sub_of(p, x, mode, (var >> 1) == 0) : -1;
      u64 pending = ballot(valid);
      while (pending) {
        const int s = read_lane(sub, __builtin_ctzll(pending));
        const bool mine = sub == s;
        const u64 m = ballot(mine);
        pending &= ~m;
        const u32 mp = wave_max_u32(mine ? (u32)p : 0u);
        const u32 mx = wave_max_u32(mine ? (u32)x : 0u);
        const u32 mr = wave_max_u32(mine ? (u32)mce_table_rows(p, x, s == MCE_SUB_MICRO ? MCE_MODE_IPX : mode) : 0u);
        const u64 words = wave_sum_u64(mine ? mce_sub_table_words(p, x, s, mode) : 0ull);
        if (lane == 0) {
          atomicAdd(&ctl->sub_count[var][s], __popcll(m));
          atomicMax(&ctl->sub_maxp[var][s], (int)mp);
          atomicMax(&ctl->sub_maxx[var][s], (int)mx);
          atomicMax(&ctl->sub_maxr[var][s], (int)mr);
          atomicAdd(&ctl->sub_words[var][s], words);
        }
      }
    }
  }
  const u64 wiso = wave_sum_u64(iso);
  const u64 whash = wave_sum_u64(iso_hash);
  const u32 wpm = wave_max_u32((u32)pmax);
  const u32 wxm = wave_max_u32((u32)xmax);
  const u32 wdm = wave_max_u32((u32)dmax);
  const u32 wl = wave_or_u32(lim);
  if (lane == 0) {
    if (wiso) {
      atomicAdd(&ctl->isolated, wiso);
      atomicAdd(&ctl->isolated_hash, whash);
    }
    atomicMax(&ctl->max_p, (int)wpm);
    atomicMax(&ctl->max_x, (int)wxm);
    atomicMax(&ctl->max_degree, (int)wdm);
    if (wl & 1u) atomicOr(&ctl->status, MCE_E_LIMIT);
    if (wl & 2u) atomicOr(&ctl->status, MCE_E_ROOTS);
  }
}

// Scatter the roots with 1 <= |P| <= MCE_MAX_P into one list per sub-class of
// the chosen mode, starting at off[sub].
__global__ __launch_bounds__(256) void k_bucket(const int* __restrict__ roots, int nroots,
                                                 const int* __restrict__ pcount, const int* __restrict__ xcount,
                                                 int mode, int micro, SubOffsets off, int* lists, u64* words,
                                                 MceCtl* ctl) {
  if (ld_relaxed(&ctl->status) != 0) return;
  const int lane = lane_id();
  const int gsize = gridDim.x * blockDim.x;
  for (int base = blockIdx.x * blockDim.x; base < nroots; base += gsize) {
    const int i = base + threadIdx.x;
    const int p = i < nroots ? pcount[i] : 0;
    const int x = i < nroots ? xcount[i] : 0;
    const bool valid = p > 0 && p <= MCE_MAX_P;
    const int sub = valid ? mce_sub_of(p, x, mode, micro != 0) : -1;
    u64 pending = ballot(valid);
    while (pending) {
      const int s = read_lane(sub, __builtin_ctzll(pending));
      const bool mine = sub == s;
      const u64 m = ballot(mine);
      pending &= ~m;
      int pos = 0;
      if (lane == 0) pos = atomicAdd(&ctl->sub_cursor[s], __popcll(m));
      pos = read_lane(pos, 0);
      if (mine) {
        lists[off.off[s] + pos + mbcnt(m)] = roots ? roots[i] : i;
        words[off.off[s] + pos + mbcnt(m)] = mce_sub_table_words(p, x, s, mode);
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
hipError_t mce_launch_validate(int n, long long nnz, const int* rp, const int* ci, MceCtl* ctl,
                               int blocks, hipStream_t s) {
  int nb = max(1, min(blocks, (n + 255) / 256));
  hipLaunchKernelGGL(k_validate_rowptr, dim3(nb), dim3(256), 0, s, n, nnz, rp, ctl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int nbw = (int)std::max(1LL, std::min((long long)blocks, ((long long)n + 3) / 4));
  hipLaunchKernelGGL(k_validate_cols, dim3(nbw), dim3(256), 0, s, n, rp, ci, ctl);
  return hipGetLastError();
}

hipError_t mce_launch_peel(int n, const int* rp, const int* ci, int* deg, int* rnd, int* core, int* alive0,
                           int* alive1, int* front0, int* front1, int* bfront0, int* bfront1, MceCtl* ctl,
                           u64 budget, int blocks, hipStream_t s) {
  void* args[] = {&n, (void*)&rp, (void*)&ci, &deg, &rnd, &core, &alive0, &alive1,
                  &front0, &front1, &bfront0, &bfront1, &ctl, &budget};
  // one block needs no grid barrier, hence no cooperative launch
  if (blocks == 1) return hipLaunchKernel((const void*)k_peel, dim3(1), dim3(PEEL_THREADS), args, 0, s);
  return hipLaunchCooperativeKernel((const void*)k_peel, dim3(blocks), dim3(PEEL_THREADS), args, 0, s);
}

// The peel's grid barrier needs every block resident: one block per CU, well
// inside the occupancy limit.
int mce_peel_max_blocks(int num_cu) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_peel, PEEL_THREADS, 0) != hipSuccess ||
      per_cu < 1)
    return 1;
  return num_cu;
}

hipError_t mce_launch_orient(int n, const int* rp, const int* ci, const int* rnd, const int* roots, int nroots,
                             int* pcount, int* xcount, MceCtl* ctl, int blocks, hipStream_t s) {
  const int nb = max(1, min(blocks, (nroots + 255) / 256));
  hipLaunchKernelGGL(k_orient, dim3(nb), dim3(256), 0, s, n, rp, ci, rnd, roots, nroots, pcount, xcount, ctl);
  return hipGetLastError();
}

hipError_t mce_launch_bucket(const int* roots, int nroots, const int* pcount, const int* xcount, int mode,
                             int micro, SubOffsets off, int* lists, u64* words, MceCtl* ctl, int blocks,
                             hipStream_t s) {
  const int nb = max(1, min(blocks, (nroots + 255) / 256));
  hipLaunchKernelGGL(k_bucket, dim3(nb), dim3(256), 0, s, roots, nroots, pcount, xcount, mode, micro, off, lists,
                     words, ctl);
  return hipGetLastError();
}

// ------------------------------------------------------------------ table offsets
// In-place exclusive prefix sum of the table sizes (u64), so that every root's
// table has a fixed heap offset before the build runs; a shared bump counter
// would take one contended atomic per root. Three passes: tiles of
// SCAN_TILE words (four per thread) scanned within a block, the tile totals
// scanned by one block, the tile prefixes added.
#define SCAN_THREADS 1024
#define SCAN_TILE (4 * SCAN_THREADS)

__device__ __forceinline__ u64 wave_incl_scan_u64(u64 v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < MCE_WAVE; d <<= 1) {
    const u64 t = __shfl_up(v, d, MCE_WAVE);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive scan of one value per thread over the block.
__device__ void block_excl_scan_u64(u64 v, u64& excl) {
  __shared__ u64 s_w[SCAN_THREADS / MCE_WAVE];
  const int lane = lane_id(), w = threadIdx.x / MCE_WAVE;
  const u64 inc = wave_incl_scan_u64(v);
  if (lane == MCE_WAVE - 1) s_w[w] = inc;
  __syncthreads();
  if (w == 0) {
    const u64 t = lane < SCAN_THREADS / MCE_WAVE ? s_w[lane] : 0ull;
    const u64 ti = wave_incl_scan_u64(t);
    if (lane < SCAN_THREADS / MCE_WAVE) s_w[lane] = ti - t;
  }
  __syncthreads();
  excl = s_w[w] + inc - v;
  __syncthreads();
}

__global__ __launch_bounds__(SCAN_THREADS) void k_scan_tiles(u64* a, int n, u64* tsum) {
  const int base = blockIdx.x * SCAN_TILE + threadIdx.x * 4;
  u64 v[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    v[q] = base + q < n ? a[base + q] : 0ull;
    sum += v[q];
  }
  u64 excl;
  block_excl_scan_u64(sum, excl);
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if (base + q < n) a[base + q] = excl;
    excl += v[q];
  }
  if (threadIdx.x == SCAN_THREADS - 1) tsum[blockIdx.x] = excl;   // the tile's total
}

__global__ __launch_bounds__(SCAN_THREADS) void k_scan_totals(u64* tsum, int nt) {
  u64 carry = 0;
  for (int b0 = 0; b0 < nt; b0 += SCAN_THREADS) {
    const int i = b0 + threadIdx.x;
    const u64 v = i < nt ? tsum[i] : 0ull;
    u64 excl;
    block_excl_scan_u64(v, excl);
    if (i < nt) tsum[i] = carry + excl;
    // block total = last thread's exclusive + its value
    __shared__ u64 s_last;
    if (threadIdx.x == SCAN_THREADS - 1) s_last = excl + v;
    __syncthreads();
    carry += s_last;
    __syncthreads();
  }
}

__global__ __launch_bounds__(SCAN_THREADS) void k_scan_add(u64* a, int n, const u64* tsum) {
  const int base = blockIdx.x * SCAN_TILE + threadIdx.x * 4;
  const u64 add = tsum[blockIdx.x];
#pragma unroll
  for (int q = 0; q < 4; q++)
    if (base + q < n) a[base + q] += add;
}

int mce_scan_temp_words(int n) { return (n + SCAN_TILE - 1) / SCAN_TILE + 1; }

hipError_t mce_launch_scan(u64* a, int n, u64* tsum, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int nt = (n + SCAN_TILE - 1) / SCAN_TILE;
  hipLaunchKernelGGL(k_scan_tiles, dim3(nt), dim3(SCAN_THREADS), 0, s, a, n, tsum);
  if (nt > 1) {   // one tile is already scanned
    hipLaunchKernelGGL(k_scan_totals, dim3(1), dim3(SCAN_THREADS), 0, s, tsum, nt);
    hipLaunchKernelGGL(k_scan_add, dim3(nt), dim3(SCAN_THREADS), 0, s, a, n, (const u64*)tsum);
  }
  return hipGetLastError();
}
