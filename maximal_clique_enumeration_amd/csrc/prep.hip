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
// ascending, and every edge present in both directions. Symmetry is checked on
// half of the edges, and on the cheap side: for an edge stored in the row of the
// endpoint that comes later in (degree, id) order, the reverse edge is searched
// in the other endpoint's row (the shorter one). Every such edge's reverse is a
// distinct stored edge from the earlier endpoint, so if both kinds are equally
// many, every edge of the second kind is such a reverse as well: the graph is
// symmetric exactly when all searches succeed and the two counts are equal.
// The entries are dealt in equal contiguous ranges, one per wavefront: the
// check of an entry (at most one binary search, in the shorter row) costs about
// the same whatever the length of its row, so equal ranges are equal work on any
// degree distribution. (Whole rows dealt to waves left single waves holding
// twenty times the mean work on an R-MAT graph, whose degrees follow the bit
// patterns of the ids.)

__device__ __forceinline__ u32 val_edge(const int* __restrict__ rp, const int* __restrict__ ci, int n, int v, int dv,
                                        int e, int b, u32& down, u32& up) {
  const int u = ci[e];
  if (u < 0 || u >= n) return 2u;                 // MCE_GRAPH_RANGE
  u32 bad = 0;
  if (u == v) return 4u;                          // MCE_GRAPH_LOOP
  if (e + 1 < b && ci[e + 1] <= u) bad |= 8u;     // MCE_GRAPH_ORDER
  const int ua = rp[u], ub = rp[u + 1];
  const int du = ub - ua;
  if (dv > du || (dv == du && v > u)) {
    down++;
    if (!csr_range_has(ci, ua, ub, v)) bad |= 16u;   // MCE_GRAPH_ASYM
  } else {
    up++;
  }
  return bad;
}

__device__ __forceinline__ void val_flush(MceCtl* ctl, u32 bad, u32 down, u32 up) {
  const u32 bb = wave_or_u32(bad);
  const u32 wd = wave_sum_u32(down);   // edges of one wave: below 2^31
  const u32 wu = wave_sum_u32(up);
  if (lane_id() == 0) {
    if (bb) atomicOr(&ctl->status, bb);
    if (wd) atomicAdd(&ctl->vdown, (u64)wd);
    if (wu) atomicAdd(&ctl->vup, (u64)wu);
  }
}

__device__ __forceinline__ int val_lane_fetch(int v, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, v); }

// The row holding entry e0 < nnz: the largest v with rp[v] <= e0, by a 64-way
// search (each step probes 64 evenly spaced row starts; rp is monotone, so the
// probes at or below e0 are a prefix of the lanes). Whole wave.
__device__ __forceinline__ int val_row_of(const int* __restrict__ rp, int n, int e0) {
  const int lane = lane_id();
  int lo = 0, hi = n;   // rp[lo] <= e0 < rp[hi]
  while (hi - lo > 1) {
    const int step = (hi - lo + MCE_WAVE - 1) / MCE_WAVE;
    const int p = lo + lane * step;
    const u64 m = ballot(p < hi && rp[p] <= e0);   // lane 0 (p = lo) always set
    lo += (63 - __builtin_clzll(m)) * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

// Wave w checks entries [w * per_wave, (w + 1) * per_wave), 64 at a time. The
// rows of a tile's entries come from one load of the next 64 row ends (lane j:
// the end of row cur + j) and a binary search over them in registers; a tile
// that spans more than 64 rows (empty rows) loads the next 64. The last block
// compares the two edge counts.
__global__ __launch_bounds__(256) void k_validate_cols(int n, long long nnz, int per_wave,
                                                        const int* __restrict__ rp, const int* __restrict__ ci,
                                                        MceCtl* ctl) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / MCE_WAVE;
  const long long e0l = (long long)wave * per_wave;
  if (ld_relaxed(&ctl->status) == 0 && e0l < nnz) {
    const int lane = lane_id();
    const int e0 = (int)e0l, e1 = (int)min(nnz, e0l + per_wave);
    u32 bad = 0, down = 0, up = 0;
    int v = val_row_of(rp, n, e0);   // row of the tile's first entry
    for (int t = e0; t < e1; t += MCE_WAVE) {
      const int e = t + lane;
      bool open = e < e1;
      int row = 0, a = 0, b = 0;
      for (int cur = v;; cur += MCE_WAVE) {
        const int cend = cur + lane + 1 <= n ? rp[cur + lane + 1] : INT_MAX;
        int k = 0;   // rows cur .. cur + k - 1 end at or before e
        for (int st = MCE_WAVE / 2; st >= 1; st >>= 1) k += val_lane_fetch(cend, k + st - 1) <= e ? st : 0;
        if (k == MCE_WAVE - 1 && val_lane_fetch(cend, MCE_WAVE - 1) <= e) k = MCE_WAVE;
        const int kb = min(k, MCE_WAVE - 1);
        const int bk = val_lane_fetch(cend, kb);
        const int ak = val_lane_fetch(cend, kb > 0 ? kb - 1 : 0);
        if (open && k < MCE_WAVE) {
          row = cur + k;
          b = bk;
          a = k > 0 ? ak : rp[cur];
          open = false;
        }
        if (!ballot(open)) break;
      }
      if (e < e1) bad |= val_edge(rp, ci, n, row, b - a, e, b, down, up);
      v = read_lane(row, MCE_WAVE - 1);   // the next tile starts in or after this row
    }
    val_flush(ctl, bad, down, up);
  }
  wait_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) {
    const u32 d = __hip_atomic_fetch_add(&ctl->vdone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == gridDim.x - 1 && ld_relaxed(&ctl->status) == 0 && ld_relaxed64(&ctl->vdown) != ld_relaxed64(&ctl->vup))
      atomicOr(&ctl->status, 16u);   // MCE_GRAPH_ASYM
  }
}

#define VAL_SMALL_N 4096
#define VAL_SMALL_NNZ 16384
__global__ __launch_bounds__(1024) void k_validate_small(int n, long long nnz, const int* __restrict__ rp,
                                                          const int* __restrict__ ci, MceCtl* ctl) {
  __shared__ u32 s_bad, s_down, s_up;
  __shared__ int s_dmax;
  const int lane = lane_id();
  if (threadIdx.x == 0) {
    s_bad = 0u;
    s_down = s_up = 0u;
    s_dmax = 0;
  }
  __syncthreads();
  u32 bad = 0;
  int dmax = 0;
  for (int v = threadIdx.x; v < n; v += blockDim.x) {
    const int a = rp[v], b = rp[v + 1];
    if (a > b || a < 0 || (long long)b > nnz) bad |= 1u;   // MCE_GRAPH_ROWPTR
    else dmax = max(dmax, b - a);
  }
  if (threadIdx.x == 0 && (rp[0] != 0 || (long long)rp[n] != nnz)) bad |= 1u;
  const u32 wb = wave_or_u32(bad);
  const u32 wm = wave_max_u32((u32)dmax);
  if (lane == 0) {
    if (wb) atomicOr(&s_bad, wb);
    if (wm) atomicMax(&s_dmax, (int)wm);
  }
  __syncthreads();
  if (s_bad == 0u) {   // uniform
    const int wave = threadIdx.x / MCE_WAVE, nwaves = blockDim.x / MCE_WAVE;
    u32 down = 0, up = 0;
    bad = 0;
    for (int v = wave; v < n; v += nwaves) {
      const int a = rp[v], b = rp[v + 1];
      for (int e = a + lane; e < b; e += MCE_WAVE) bad |= val_edge(rp, ci, n, v, b - a, e, b, down, up);
    }
    const u32 bb = wave_or_u32(bad), wd = wave_sum_u32(down), wu = wave_sum_u32(up);
    if (lane == 0) {
      if (bb) atomicOr(&s_bad, bb);
      if (wd) atomicAdd(&s_down, wd);
      if (wu) atomicAdd(&s_up, wu);
    }
    __syncthreads();
    if (threadIdx.x == 0 && s_bad == 0u && s_down != s_up) s_bad = 16u;   // MCE_GRAPH_ASYM
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (s_bad) atomicOr(&ctl->status, s_bad);
    if (s_dmax) atomicMax(&ctl->max_degree, s_dmax);
  }
}

// ------------------------------------------------------------------ k-core peel
// Grid-wide barrier for a cooperative launch, without agent-scope fences (their
// L2 write-back / invalidate serialises when hundreds of blocks issue them).
// Everything the peel passes between blocks is read and written with
// agent-scope relaxed atomics, which are performed at the device coherence
// point; the barrier only has to order them: each block waits until its own
// memory operations completed, then arrives. Two levels, because atomics on one
// address serialise (256 arrivals on one counter: 3.9 us a barrier; this way
// 1.8 us): block b arrives on the counter of group b mod 16; the block that
// completes its group counts the group complete, and the block that completes
// the last group releases the barrier on a line that nobody adds to. Counters
// only grow (zeroed with the control block before the launch): barrier e of the
// launch is complete once a group counter reaches e times the group's size,
// so no block resets anything or opens a generation. Bounded: past the
// deadline it flags MCE_E_TIMEOUT and lets the block go; the caller checks the
// flag after every barrier.
__device__ __forceinline__ void grid_sync(MceCtl* ctl, u64 deadline, u32& epoch, bool solo = false) {
  wait_stores_complete();
  __syncthreads();
  if (gridDim.x > 1 && !solo) {
    if (threadIdx.x == 0) {
      epoch++;
      const u32 ng = min(gridDim.x, (u32)MCE_BAR_GROUPS);
      const u32 g = blockIdx.x % ng;
      const u32 gsize = (gridDim.x - g + ng - 1) / ng;   // blocks b with b mod ng == g
      u32* done = &ctl->bar[0];
      u32* rel = &ctl->bar[MCE_BAR_STRIDE];
      u32* gc = &ctl->bar[(2 + g) * MCE_BAR_STRIDE];
      bool last = false;
      if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == epoch * gsize &&
          __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == epoch * ng) {
        st_relaxed(rel, epoch);
        last = true;
      }
      u32 spins = 0;
      while (!last && ld_relaxed(rel) < epoch) {
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
#ifndef PEEL_LDS_N
#define PEEL_LDS_N 4096   // one-block peels of at most this many vertices keep degrees and rounds in LDS
#endif
#define PEEL_LPER 8                            // entries per thread and tile of a level pass
// The tail: once at most PEEL_TT vertices remain, each with at most
// PEEL_TMAXDEG live neighbours, and their live entries fill at most tcap
// 16-bit words, block 0 finishes on the residual graph compacted to local ids
// (0xFFFF pads rows and is no local id), with the degrees in its LDS.
#define PEEL_TT 65535
#define PEEL_TMAXDEG 32767
#define PEEL_TLONG 8192     // rows longer than this (CSR entries) are compacted in spans by every wavefront
#define PEEL_TSPAN 1024     // CSR entries of a span, and of a step of a shorter row (16 per lane)
#define PEEL_TPER (PEEL_TSPAN / MCE_WAVE)
#ifndef PEEL_TQ
#define PEEL_TQ 2           // tail rounds: 16-byte loads per lane in flight
#endif
#ifndef PEEL_TFCAP
#define PEEL_TFCAP 2048     // frontier entries of a tail round kept in LDS; more go to a global list
#endif
#define PEEL_TPOOL ((PEEL_TT + 1) / 2 + PEEL_TFCAP)   // LDS words of the tail: packed degrees, two lists
// Entries a remaining vertex of degree d and CSR row length len takes in the
// compacted graph: its live neighbours, padded to a multiple of 8 (one 16-byte
// load per lane reads 8); a row compacted in spans pads every span.
__device__ __forceinline__ long long tail_budget(int d, int len) {
  const int extra = len > PEEL_TLONG ? 7 * ((len + PEEL_TSPAN - 1) / PEEL_TSPAN) : 0;
  return (long long)((d + extra + 7) & ~7);
}
#define PEEL_LTILE (PEEL_LPER * PEEL_THREADS)   // entries per tile

// Appends the lanes with `in` set to the next frontier: the regular list, or
// the big list for vertices of degree > PEEL_BIG, whose CSR row lengths are
// also summed (the rows of the others are short by definition). Whole wave.
template <int S>
__device__ __forceinline__ void peel_append(bool in, int v, const int* __restrict__ rp, int* fr, int* fsize,
                                            int* bfr, int* bsize, int* bedge) {
  const int lane = lane_id();
  const int len = in ? rp[v + 1] - rp[v] : 0;
  const bool big = len > PEEL_BIG;
  const u64 mr = ballot(in && !big);
  const u64 mb = ballot(big);
  int pr = 0, pb = 0;
  if (lane == 0 && mr) pr = padd<S>(fsize, __popcll(mr));
  if (mb) {
    const u32 es = wave_sum_u32(big ? (u32)len : 0u);   // distinct rows: at most nnz
    if (lane == 0) {
      pb = padd<S>(bsize, __popcll(mb));
      padd<S>(bedge, (int)es);
    }
  }
  pr = read_lane(pr, 0);
  pb = read_lane(pb, 0);
  if (in && !big) pst<S>(&fr[pr + mbcnt(mr)], v);
  if (big) pst<S>(&bfr[pb + mbcnt(mb)], v);
}

// A neighbour's degree is taken only while it is still present. Its round is
// read with a plain load: a stale copy can only show -1 (present), and taking a
// degree from a removed vertex is harmless (it has degree <= k at its removal
// and only loses more, so it never falls from k + 1 again; its degree is not
// read any more). Skipping the removed ones saves about half of the returning
// atomics, which bound the peel.
#ifndef PEEL_FILTER
#define PEEL_FILTER 1
#endif
__device__ __forceinline__ bool peel_present(const int* rnd, int u) {
  return !PEEL_FILTER || rnd[u] < 0;
}

// One span of a removed vertex's row [base, min(base + PEEL_SPAN, b)): take one
// degree from each present neighbour (all four 64-edge pieces in flight
// together). A neighbour that falls from k + 1 to k joins the next round.
template <int S>
__device__ __forceinline__ void peel_span(int base, int b, int k, const int* __restrict__ rp,
                                          const int* __restrict__ ci, const int* rnd, int* deg, int* nx, int* nxs,
                                          int* bnx, int* bnxs, int* bnxe) {
  const int lane = lane_id();
  int u[4];
  bool ok[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int e = base + q * MCE_WAVE + lane;
    ok[q] = e < b;
    u[q] = ok[q] ? ci[e] : 0;
  }
#pragma unroll
  for (int q = 0; q < 4; q++) ok[q] = ok[q] && peel_present(rnd, u[q]);
  bool joins[4];
#pragma unroll
  for (int q = 0; q < 4; q++) joins[q] = ok[q] && padd<S>(&deg[u[q]], -1) == k + 1;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if (ballot(joins[q])) peel_append<S>(joins[q], u[q], rp, nx, nxs, bnx, bnxs, bnxe);
  }
}

// Appends the joiners of up to four loads at once (lane l of load q joins when
// bit l of jm[q] is set; its vertex is u[q]): one device-scope atomic per list
// (regular, big) for all of them. Whole wave.
template <int S>
__device__ __forceinline__ void peel_append4(const u64 (&jm)[4], const int (&u)[4], const int* __restrict__ rp,
                                             int* fr, int* fsize, int* bfr, int* bsize, int* bedge) {
  const int lane = lane_id();
  if (!(jm[0] | jm[1] | jm[2] | jm[3])) return;
  u64 mr[4], mb[4];
  int nr = 0, nbg = 0;
  u32 eb = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const bool in = (jm[q] >> lane) & 1ull;
    const int len = in ? rp[u[q] + 1] - rp[u[q]] : 0;
    const bool big = len > PEEL_BIG;
    mr[q] = ballot(in && !big);
    mb[q] = ballot(big);
    nr += __popcll(mr[q]);
    nbg += __popcll(mb[q]);
    eb += big ? (u32)len : 0u;
  }
  const u32 es = nbg ? wave_sum_u32(eb) : 0u;
  int pr = 0, pb = 0;
  if (lane == 0) {
    if (nr) pr = padd<S>(fsize, nr);
    if (nbg) {
      pb = padd<S>(bsize, nbg);
      padd<S>(bedge, (int)es);
    }
  }
  pr = read_lane(pr, 0);
  pb = read_lane(pb, 0);
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if ((mr[q] >> lane) & 1ull) pst<S>(&fr[pr + mbcnt(mr[q])], u[q]);
    if ((mb[q] >> lane) & 1ull) pst<S>(&bfr[pb + mbcnt(mb[q])], u[q]);
    pr += __popcll(mr[q]);
    pb += __popcll(mb[q]);
  }
}

// The rows of a group of up to 64 frontier vertices (lane t: vertex t's CSR
// row [a, a + len), incl = the lanes' inclusive prefix of the lengths, E =
// all of them), their entries taken 64 at a time whichever rows they fall in
// (lane l of step s takes entry 64 s + l, its row found by a binary search
// over the lanes' prefix), four steps in flight: each present neighbour loses
// one degree, and one that falls from k + 1 to k joins the next round. Whole
// wave.
// ONE: the group is one vertex (lane 0's row), found without a search.
template <int S, bool ONE>
__device__ __forceinline__ void peel_group(int a, int incl, int E, int k, const int* __restrict__ rp,
                                           const int* __restrict__ ci, const int* rnd, int* deg, int* nx, int* nxs,
                                           int* bnx, int* bnxs, int* bnxe) {
  const int lane = lane_id();
  const int a0 = read_lane(a, 0);
  for (int e0 = 0; e0 < E; e0 += 4 * MCE_WAVE) {
    int u[4];
    bool ok[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int e = e0 + q * MCE_WAVE + lane;
      int pos = a0 + e;
      if (!ONE) {
        // (every lane takes part in each shuffle: one that sat out would read
        // 0 from the lanes that do)
        int t = 0;
#pragma unroll
        for (int step = 32; step > 0; step >>= 1) {
          const int v = __shfl(incl, t + step - 1);
          if (v <= e) t += step;
        }
        const int tt = min(t, MCE_WAVE - 1);
        const int at = __shfl(a, tt);
        const int pre = __shfl(incl, max(tt - 1, 0));
        pos = at + e - (tt > 0 ? pre : 0);
      }
      ok[q] = e < E;
      u[q] = ok[q] ? ci[pos] : 0;
    }
#pragma unroll
    for (int q = 0; q < 4; q++) ok[q] = ok[q] && peel_present(rnd, u[q]);
    u64 jm[4];
#pragma unroll
    for (int q = 0; q < 4; q++) jm[q] = ballot(ok[q] && padd<S>(&deg[u[q]], -1) == k + 1);
    peel_append4<S>(jm, u, rp, nx, nxs, bnx, bnxs, bnxe);
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
  int* sc;      // block 0's LDS counter slots while it runs a segment (12)
  int4* sfr;   // block 0's LDS frontier lists while it runs a segment: (v, row start, row end)
  // the residual graph compacted for block 0 (peel_tail_build, peel_tail_rounds)
  unsigned short* tcol;   // rows of 16-bit local ids, each padded to a multiple of 8 entries
  long long tcap;         // entries tcol holds; 0: no compaction, the grid peels to the end
  int* tcrow;             // row starts, PEEL_TT + 1
  u32* pool;              // block 0's LDS in the tail: packed degrees and frontier lists
  unsigned char* snap;    // split peel (or NULL): 1 for every vertex still present at the hand-over
  // ping-pong buffers by parity (selects, not indexed arrays: no scratch memory)
  __device__ int* alive(int i) const { return (i & 1) ? alive1 : alive0; }
  __device__ int* front(int i) const { return (i & 1) ? front1 : front0; }
  __device__ int* bfront(int i) const { return (i & 1) ? bfront1 : bfront0; }
};

struct PeelState {
  int cur, nf, nb, k, r, na;
  int ph;               // slot of the pending frontier's sizes
  int fe;               // the pending frontier's CSR row lengths summed
  int ae;               // the remaining list's CSR row lengths summed (at its level pass)
  int tdmax;            // its largest degree, and
  long long tsize;      // its compacted size in entries (both when it is short enough to compact)
  bool level_known;     // the level's remaining list and k are known, its first round is not built
  u32 epoch;            // grid barriers passed (thread 0 of each block)
  u32 seg;              // segments of tiny rounds handed from the grid to block 0
  u64 tb, tl, tr, tm;   // first block's thread 0: barrier, level, round ticks; last mark
};

#define PEEL_MARK(acc)                \
  if (timer) {                        \
    const u64 t = wall_clock64();     \
    st.acc += t - st.tm;              \
    st.tm = t;                        \
  }

// Who runs the rounds: the whole grid at agent scope, or block 0 alone at
// workgroup scope once few vertices remain (the others left). Tiny rounds in
// between are run by block 0 too (peel_seg).
#define PEEL_GRID 0
#define PEEL_ALONE 2
// What peel_rounds returns.
#define PEEL_DONE 0
#define PEEL_TIMEOUT (-1)
#define PEEL_TO_ALONE 1   // at most PEEL_SOLO vertices with PEEL_SOLO_EDGES edges remain
#define PEEL_TO_SEG 2     // the next round removes at most PEEL_TINY vertices, big ones with PEEL_SEG_EDGES edges
#define PEEL_TO_GRID 3    // block 0 hands back a larger round or a level pass
#define PEEL_TO_TAIL 4    // few enough vertices remain to compact the residual graph for block 0
#ifndef PEEL_TINY
#define PEEL_TINY 32
#endif
static_assert(PEEL_TINY <= MCE_WAVE, "a segment round's frontier fits one wavefront's lanes");
#ifndef PEEL_SEG_EDGES
#define PEEL_SEG_EDGES 16384
#endif
#ifndef PEEL_SOLO_EDGES
#define PEEL_SOLO_EDGES 262144
#endif
__device__ __forceinline__ bool peel_few_left(const PeelState& st) {
  return st.na <= PEEL_SOLO && st.ae <= PEEL_SOLO_EDGES;
}

// Rounds of the peel (see k_peel). `wave`/`nwaves` index the waves taking part.
//
// Frontier sizes rotate over three slots, one step (level pass, first-round
// scan or round: the work between two barriers) at a time. The step after slot
// ph was filled appends the next frontier to slot ph + 1 and clears slot
// ph + 2. A barrier lets blocks go at different times, so a slow block may
// still be reading slot ph while a fast one works on the next step; slot ph + 2
// was last read before the previous barrier, which every block has passed.
// The remaining-list sizes and minima are kept per list parity for the same
// reason: they are reset one level after they were read.
// (always inlined: as a call, its state structures would live in scratch memory)
template <int S, int MODE>
__device__ __forceinline__ int peel_rounds(const PeelArgs& A, PeelState& st, int wave, int nwaves, bool timer) {
  const int lane = lane_id();
  constexpr bool BLOCK = MODE != PEEL_GRID;   // block 0 alone: workgroup barriers
  const bool lead = BLOCK ? threadIdx.x == 0 : (blockIdx.x == 0 && threadIdx.x == 0);
  MceCtl* ctl = A.ctl;
  const int* rp = A.rp;
  int* fs = ctl->fsize;
  int* bs = ctl->bsize;
  int* be = ctl->bedge;
  for (;;) {
    if (st.nf == 0 && st.nb == 0) {
      if (!st.level_known) {
        // New level: compact the remaining list and find the smallest remaining
        // degree. Every remaining vertex has degree > k, so the next level is
        // k + 1 exactly when some vertex has degree k + 1: those vertices, the
        // level's first round, are collected in the same pass.
        const int p1 = (st.ph + 1) % 3, p2 = (st.ph + 2) % 3;
        if (lead) {
          pst<S>(&fs[p2], 0);
          pst<S>(&bs[p2], 0);
          pst<S>(&be[p2], 0);
        }
        const int* src = A.alive(st.cur);
        int* dst = A.alive(st.cur ^ 1);
        const int kn = st.k + 1;
        // the kept rows' lengths decide whether block 0 may finish alone; they
        // cost a gather per vertex, so they are summed only once the list is short
        const bool sum_rows = st.na <= 8 * PEEL_SOLO;
        // the kept vertices' largest degree and compacted size decide whether
        // block 0 can finish on the compacted residual graph
        const bool sum_tail = MODE == PEEL_GRID && A.tcap > 0 && st.na <= 2 * PEEL_TT;
        // Tiles of PEEL_LTILE entries per block: one atomic on the shared list
        // size per tile, and one per block for the minimum and the row sum
        // (same-address device-scope atomics serialise; one per wavefront and
        // 64 entries made the early levels of a 4M-vertex graph cost 1 ms each).
        __shared__ int s_lv[PEEL_THREADS / MCE_WAVE + 1];
        __shared__ int s_mn;
        __shared__ u32 s_rows;
        __shared__ int s_tmax;
        __shared__ unsigned long long s_tsum;
        const int bw = threadIdx.x / MCE_WAVE, nbw = blockDim.x / MCE_WAVE;
        const int blk = BLOCK ? 0 : (int)blockIdx.x, nblk = BLOCK ? 1 : (int)gridDim.x;
        if (threadIdx.x == 0) {
          s_mn = 0x7FFFFFFF;
          s_rows = 0u;
          s_tmax = 0;
          s_tsum = 0ull;
        }
        int mn = 0x7FFFFFFF;
        u32 rows = 0;   // CSR row lengths of the kept vertices (at most nnz in all)
        long long tsum = 0;
        int tmax = 0;
        for (int tb = blk * PEEL_LTILE; tb < st.na; tb += nblk * PEEL_LTILE) {   // uniform in the block
          bool keep[PEEL_LPER], first[PEEL_LPER];
          int v[PEEL_LPER];
#pragma unroll
          for (int q = 0; q < PEEL_LPER; q++) {
            const int i = tb + q * PEEL_THREADS + (int)threadIdx.x;
            keep[q] = first[q] = false;
            v[q] = 0;
            if (i < st.na) v[q] = pld<S>(&src[i]);
          }
          // a vertex's round and degree are loaded together (the degree of a
          // removed one is not used)
          int dvq[PEEL_LPER];
#pragma unroll
          for (int q = 0; q < PEEL_LPER; q++) {
            const int i = tb + q * PEEL_THREADS + (int)threadIdx.x;
            dvq[q] = 0;
            if (i < st.na) {
              keep[q] = pld<S>(&A.rnd[v[q]]) < 0;
              dvq[q] = pld<S>(&A.deg[v[q]]);
            }
          }
#pragma unroll
          for (int q = 0; q < PEEL_LPER; q++) {
            if (keep[q]) {
              const int dv = dvq[q];
              mn = min(mn, dv);
              first[q] = dv <= kn;
              if (sum_rows || sum_tail) {
                const int len = rp[v[q] + 1] - rp[v[q]];
                if (sum_rows) rows += (u32)len;
                if (sum_tail) {
                  tsum += tail_budget(dv, len);
                  tmax = max(tmax, dv);
                }
              }
            }
          }
          u64 m[PEEL_LPER];
          int cnt = 0;
#pragma unroll
          for (int q = 0; q < PEEL_LPER; q++) {
            m[q] = ballot(keep[q]);
            cnt += __popcll(m[q]);
          }
          if (lane == 0) s_lv[bw] = cnt;
          __syncthreads();
          if (threadIdx.x == 0) {
            int run = 0;
            for (int w = 0; w < nbw; w++) {
              const int c = s_lv[w];
              s_lv[w] = run;
              run += c;
            }
            s_lv[nbw] = run ? padd<S>(&ctl->asize[st.cur ^ 1], run) : 0;
          }
          __syncthreads();
          int pos = s_lv[nbw] + s_lv[bw];
#pragma unroll
          for (int q = 0; q < PEEL_LPER; q++) {
            if (keep[q]) pst<S>(&dst[pos + mbcnt(m[q])], v[q]);
            pos += __popcll(m[q]);
          }
          // the tile's first-round vertices: one append per list and wave for
          // all of the tile's entries (each is a device-scope round trip)
          {
            u64 mr[PEEL_LPER], mbg[PEEL_LPER];
            int nr = 0, nbg = 0;
            u32 eb = 0;
#pragma unroll
            for (int q = 0; q < PEEL_LPER; q++) {
              const int len = first[q] ? rp[v[q] + 1] - rp[v[q]] : 0;
              const bool big = len > PEEL_BIG;
              mr[q] = ballot(first[q] && !big);
              mbg[q] = ballot(big);
              nr += __popcll(mr[q]);
              nbg += __popcll(mbg[q]);
              eb += big ? (u32)len : 0u;
            }
            if (nr + nbg > 0) {
              const u32 es = nbg ? wave_sum_u32(eb) : 0u;
              int pr = 0, pb = 0;
              if (lane == 0) {
                if (nr) pr = padd<S>(&fs[p1], nr);
                if (nbg) {
                  pb = padd<S>(&bs[p1], nbg);
                  padd<S>(&be[p1], (int)es);
                }
              }
              pr = read_lane(pr, 0);
              pb = read_lane(pb, 0);
              int* fr = A.front(st.r);
              int* bfr = A.bfront(st.r);
#pragma unroll
              for (int q = 0; q < PEEL_LPER; q++) {
                if ((mr[q] >> lane) & 1ull) pst<S>(&fr[pr + mbcnt(mr[q])], v[q]);
                if ((mbg[q] >> lane) & 1ull) pst<S>(&bfr[pb + mbcnt(mbg[q])], v[q]);
                pr += __popcll(mr[q]);
                pb += __popcll(mbg[q]);
              }
            }
          }
          __syncthreads();   // s_lv is filled again for the next tile
        }
        const int wmn = wave_min_i32_nonneg(mn);
        if (lane == 0 && wmn != 0x7FFFFFFF) atomicMin(&s_mn, wmn);
        if (sum_rows) {
          const u32 wrows = wave_sum_u32(rows);
          if (lane == 0 && wrows) atomicAdd(&s_rows, wrows);
        }
        if (sum_tail) {
          const u64 wts = wave_sum_u64((u64)tsum);
          const u32 wtm = wave_max_u32((u32)tmax);
          if (lane == 0) {
            if (wts) atomicAdd(&s_tsum, (unsigned long long)wts);
            if (wtm) atomicMax(&s_tmax, (int)wtm);
          }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
          if (s_mn != 0x7FFFFFFF) pmin<S>(&ctl->min_deg[st.cur ^ 1], s_mn);
          if (s_rows) padd<S>(&ctl->asum[st.cur ^ 1], (int)s_rows);
          if (s_tsum) __hip_atomic_fetch_add(&ctl->tsum[st.cur ^ 1], (u64)s_tsum, __ATOMIC_RELAXED, S);
          if (s_tmax) __hip_atomic_fetch_max(&ctl->tmax[st.cur ^ 1], s_tmax, __ATOMIC_RELAXED, S);
        }
        PEEL_MARK(tl);
        grid_sync(ctl, A.deadline, st.epoch, BLOCK);
        PEEL_MARK(tb);
        st.cur ^= 1;
        st.ph = p1;
        const u32 status = ld_relaxed(&ctl->status);
        st.na = pld<S>(&ctl->asize[st.cur]);
        const int kmin = pld<S>(&ctl->min_deg[st.cur]);   // no remaining vertex: k stays the degeneracy
        st.ae = sum_rows ? pld<S>(&ctl->asum[st.cur]) : 0x7FFFFFFF;
        st.tsize = sum_tail ? (long long)__hip_atomic_load(&ctl->tsum[st.cur], __ATOMIC_RELAXED, S) : 0x7FFFFFFFFFFFFFFFll;
        st.tdmax = sum_tail ? pld<S>(&ctl->tmax[st.cur]) : 0x7FFFFFFF;
        st.nf = pld<S>(&fs[p1]);
        st.nb = pld<S>(&bs[p1]);
        st.fe = pld<S>(&be[p1]);
        if (status & MCE_E_TIMEOUT) return PEEL_TIMEOUT;
        if (st.na == 0) return PEEL_DONE;
        const bool built = st.nf + st.nb > 0;   // then kmin == k + 1
        st.k = built ? kn : kmin;
        // few enough vertices with few enough live entries: compact the
        // residual graph, and block 0 finishes on it (the level's first round
        // is found again there from the degrees)
        if (MODE == PEEL_GRID && gridDim.x > 1 && sum_tail && st.na <= PEEL_TT && st.tdmax <= PEEL_TMAXDEG &&
            st.tsize <= A.tcap)
          return PEEL_TO_TAIL;
        if (MODE == PEEL_GRID && gridDim.x > 1 && peel_few_left(st)) {
          st.level_known = !built;
          return PEEL_TO_ALONE;
        }
        if (built) continue;
      }
      st.level_known = false;
      // the level's first round: every remaining vertex of degree <= k
      const int p1 = (st.ph + 1) % 3, p2 = (st.ph + 2) % 3;
      if (lead) {
        pst<S>(&fs[p2], 0);
        pst<S>(&bs[p2], 0);
        pst<S>(&be[p2], 0);
      }
      const int* al = A.alive(st.cur);
      for (int base = wave * MCE_WAVE; base < st.na; base += nwaves * MCE_WAVE) {
        const int i = base + lane;
        bool in = false;
        int v = 0;
        if (i < st.na) {
          v = pld<S>(&al[i]);
          in = pld<S>(&A.deg[v]) <= st.k;
        }
        peel_append<S>(in, v, rp, A.front(st.r), &fs[p1], A.bfront(st.r), &bs[p1], &be[p1]);
      }
      PEEL_MARK(tl);
      grid_sync(ctl, A.deadline, st.epoch, BLOCK);
      PEEL_MARK(tb);
      st.ph = p1;
      const u32 status2 = ld_relaxed(&ctl->status);
      st.nf = pld<S>(&fs[p1]);
      st.nb = pld<S>(&bs[p1]);
      st.fe = pld<S>(&be[p1]);
      if (status2 & MCE_E_TIMEOUT) return PEEL_TIMEOUT;
    }
    if (MODE == PEEL_GRID && gridDim.x > 1 && st.nf + st.nb <= PEEL_TINY && st.fe <= PEEL_SEG_EDGES)
      return PEEL_TO_SEG;
    // round r: remove the frontier, take one degree from each neighbour
    const int r = st.r, k = st.k;
    const int p1 = (st.ph + 1) % 3, p2 = (st.ph + 2) % 3;
    if (lead) {
      pst<S>(&fs[p2], 0);
      pst<S>(&bs[p2], 0);
      pst<S>(&be[p2], 0);
      // the other list's size, row sum and minimum were read a level ago
      pst<S>(&ctl->asize[st.cur ^ 1], 0);
      pst<S>(&ctl->asum[st.cur ^ 1], 0);
      pst<S>(&ctl->min_deg[st.cur ^ 1], 0x7FFFFFFF);
      pst<S>(&ctl->tmax[st.cur ^ 1], 0);
      __hip_atomic_store(&ctl->tsum[st.cur ^ 1], 0ull, __ATOMIC_RELAXED, S);
    }
    const int* fr = A.front(r);
    const int* bfr = A.bfront(r);
    int* nx = A.front(r + 1);
    int* nxs = &fs[p1];
    int* bnx = A.bfront(r + 1);
    int* bnxs = &bs[p1];
    int* bnxe = &be[p1];
    // vertices of small degree (rows of at most PEEL_BIG entries): groups of
    // G per wave, G = 1 while there are at most as many as waves (a vertex's
    // row gets all 64 lanes), up to 64 on the large rounds at the start of a
    // level (one lane per vertex would leave most lanes idle on short rows,
    // and one vertex per wave at a time made such rounds a chain of hundreds
    // of dependent round trips)
    {
      const int G = min(MCE_WAVE, (st.nf + nwaves - 1) / nwaves);
      for (int g0 = wave * G; g0 < st.nf; g0 += nwaves * G) {
        int a = 0, len = 0;
        if (lane < G && g0 + lane < st.nf) {
          const int v = pld<S>(&fr[g0 + lane]);
          pst<S>(&A.rnd[v], r);
          A.core[v] = k;
          a = rp[v];
          len = rp[v + 1] - a;
        }
        int incl = len;
#pragma unroll
        for (int o = 1; o < MCE_WAVE; o <<= 1) {
          const int t = __shfl_up(incl, o);
          if (lane >= o) incl += t;
        }
        const int E = read_lane(incl, MCE_WAVE - 1);
        if (G == 1) peel_group<S, true>(a, incl, E, k, rp, A.ci, A.rnd, A.deg, nx, nxs, bnx, bnxs, bnxe);
        else peel_group<S, false>(a, incl, E, k, rp, A.ci, A.rnd, A.deg, nx, nxs, bnx, bnxs, bnxe);
      }
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
          peel_span<S>(a + c * PEEL_SPAN, b, k, rp, A.ci, A.rnd, A.deg, nx, nxs, bnx, bnxs, bnxe);
      }
    }
    PEEL_MARK(tr);
    grid_sync(ctl, A.deadline, st.epoch, BLOCK);
    PEEL_MARK(tb);
    st.ph = p1;
    const u32 status = ld_relaxed(&ctl->status);
    st.nf = pld<S>(nxs);
    st.nb = pld<S>(bnxs);
    st.fe = pld<S>(bnxe);
    st.r++;
    if (status & MCE_E_TIMEOUT) return PEEL_TIMEOUT;
  }
}

// Block 0's workgroup barrier over LDS only: its global stores (rounds and core
// numbers, spilled frontier entries) are not waited for until it hands back.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A segment of tiny rounds, run by block 0 while the other blocks wait. The
// frontier (vertices of any degree) is kept in LDS as (v, row start, row end),
// its counts in LDS slots (the same three-slot rotation as the grid's); the
// rows of a round are cut into 64-edge pieces dealt over all of block 0's
// waves, so that a round of a few thousand edges takes about one dependent
// chain of memory operations. The only global operations are the edge loads,
// the degree decrements, the row bounds of the vertices that join the next
// round, and stores nobody reads before the hand-back; joiners past the first
// PEEL_TINY go straight to the global lists. Returns PEEL_TO_GRID (a larger
// round, whose LDS entries it has moved to the global lists, or a level pass)
// or PEEL_TO_ALONE.
__device__ __forceinline__ int peel_seg(const PeelArgs& A, PeelState& st, int wave, int nwaves, bool timer) {
  __shared__ int s_split[2];
  const int lane = lane_id();
  const int* __restrict__ rp = A.rp;
  const int* __restrict__ ci = A.ci;
  // LDS slots: entries of the LDS list, their row lengths summed, and joiners
  // past the list that went to the global small / big lists
  int* c_n = A.sc;
  int* c_e = A.sc + 3;
  int* c_gs = A.sc + 6;
  int* c_gb = A.sc + 9;
  {
    const int* fr = A.front(st.r);
    const int* bfr = A.bfront(st.r);
    const int tot = st.nf + st.nb;
    if (threadIdx.x < 12) A.sc[threadIdx.x] = 0;
    lds_barrier();
    for (int i = threadIdx.x; i < tot; i += blockDim.x) {
      const int v = i < st.nf ? pld<SA>(&fr[i]) : pld<SA>(&bfr[i - st.nf]);
      const int a = rp[v], b = rp[v + 1];
      A.sfr[i] = make_int4(v, a, b, 0);
      if (b - a > PEEL_BIG) atomicAdd(&A.sc[3], b - a);   // big rows' lengths, in slot 0 of the edge count
    }
    lds_barrier();
    st.fe = A.sc[3];
    if (st.fe > PEEL_SEG_EDGES) return PEEL_TO_GRID;   // rows too long: the grid takes the round
    st.nf = tot;   // in a segment nf counts the LDS entries, of any degree
    st.nb = 0;
  }
  int lp = 0;
  for (int j = 0;; j++) {
    const int r = st.r, k = st.k;
    const int p1 = (lp + 1) % 3, p2 = (lp + 2) % 3;
    if (threadIdx.x == 0) {
      c_n[p2] = 0;
      c_e[p2] = 0;
      c_gs[p2] = 0;
      c_gb[p2] = 0;
    }
    // the two LDS lists alternate by round (selects: no indexed private array)
    const int4* cur = (j & 1) ? A.sfr + PEEL_TINY : A.sfr;
    int4* nxt = (j & 1) ? A.sfr : A.sfr + PEEL_TINY;
    int* gnx = A.front(r + 1);
    int* gbnx = A.bfront(r + 1);
    // lane t of every wave holds entry t (nf <= PEEL_TINY <= 64); the entries'
    // rows are cut into 64-edge pieces, dealt round-robin over the waves
    int4 e = make_int4(0, 0, 0, 0);
    if (lane < st.nf) e = cur[lane];
    const int cnt = lane < st.nf ? (e.z - e.y + MCE_WAVE - 1) / MCE_WAVE : 0;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < MCE_WAVE; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int total = read_lane(incl, MCE_WAVE - 1);
    if (wave == 0 && lane < st.nf) {
      pst<SA>(&A.rnd[e.x], r);
      A.core[e.x] = k;
    }
    for (int p0 = wave; p0 < total; p0 += 4 * nwaves) {
      int u[4];
      bool ok[4], joins[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int pc = p0 + q * nwaves;
        ok[q] = false;
        u[q] = 0;
        if (pc < total) {
          const int t = __popcll(ballot(incl <= pc));   // the entry holding piece pc
          const int first = read_lane(incl, t) - read_lane(cnt, t);
          const int ed = read_lane(e.y, t) + (pc - first) * MCE_WAVE + lane;
          ok[q] = ed < read_lane(e.z, t);
          u[q] = ok[q] ? ci[ed] : 0;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; q++) ok[q] = ok[q] && peel_present(A.rnd, u[q]);
#pragma unroll
      for (int q = 0; q < 4; q++) joins[q] = ok[q] && padd<SA>(&A.deg[u[q]], -1) == k + 1;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        if (!ballot(joins[q])) continue;
        int a = 0, b = 0;
        if (joins[q]) {
          a = rp[u[q]];
          b = rp[u[q] + 1];
        }
        const u64 mj = ballot(joins[q]);
        int pos = 0;
        if (lane == 0) pos = atomicAdd(&c_n[p1], __popcll(mj));
        pos = read_lane(pos, 0) + mbcnt(mj);
        const bool inl = joins[q] && pos < PEEL_TINY;
        if (inl) nxt[pos] = make_int4(u[q], a, b, 0);
        const u32 le = wave_sum_u32(inl && b - a > PEEL_BIG ? (u32)(b - a) : 0u);
        if (lane == 0 && le) atomicAdd(&c_e[p1], (int)le);
        const bool ov = joins[q] && !inl;   // past the LDS list: straight to the global lists
        if (ballot(ov)) {
          const bool big = ov && b - a > PEEL_BIG;
          const u64 ms = ballot(ov && !big), mb = ballot(big);
          int ps = 0, pb = 0;
          if (lane == 0 && ms) ps = atomicAdd(&c_gs[p1], __popcll(ms));
          if (lane == 0 && mb) pb = atomicAdd(&c_gb[p1], __popcll(mb));
          ps = read_lane(ps, 0);
          pb = read_lane(pb, 0);
          if (ov && !big) pst<SA>(&gnx[ps + mbcnt(ms)], u[q]);
          if (big) pst<SA>(&gbnx[pb + mbcnt(mb)], u[q]);
        }
      }
    }
    PEEL_MARK(tr);
    lds_barrier();
    PEEL_MARK(tb);
    const int tot = c_n[p1];
    const int gs = c_gs[p1], gb = c_gb[p1];
    st.fe = c_e[p1];
    st.r++;
    lp = p1;
    if (tot == 0) {
      st.nf = 0;
      st.nb = 0;
      return peel_few_left(st) ? PEEL_TO_ALONE : PEEL_TO_GRID;
    }
    if (tot > PEEL_TINY || st.fe > PEEL_SEG_EDGES) {
      // the grid takes this round: the LDS entries join the global lists after the spilled ones
      if (wave == 0) {
        const bool valid = lane < min(tot, PEEL_TINY);
        const int4 e2 = valid ? nxt[lane] : make_int4(0, 0, 0, 0);
        const bool big = valid && e2.z - e2.y > PEEL_BIG;
        const u64 ms = ballot(valid && !big), mb = ballot(big);
        if (valid && !big) pst<SA>(&gnx[gs + mbcnt(ms)], e2.x);
        if (big) pst<SA>(&gbnx[gb + mbcnt(mb)], e2.x);
        if (lane == 0) {
          s_split[0] = gs + __popcll(ms);
          s_split[1] = gb + __popcll(mb);
        }
      }
      lds_barrier();
      st.nf = s_split[0];
      st.nb = s_split[1];
      return PEEL_TO_GRID;
    }
    st.nf = tot;
    st.nb = 0;
  }
}

// Block 0 hands a segment back (every thread of block 0 calls this): its stores
// complete, then, once
// every waiting block has arrived (and so has read what the barrier before the
// segment published), the control block's counters are set for the grid's next
// step, then the state goes out, then the generation counter.
__device__ __forceinline__ int peel_hand_back(MceCtl* ctl, const PeelState& st, int res, u64 deadline) {
  __shared__ int s_res;
  wait_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) {
    const u32 want = st.seg * (gridDim.x - 1);
    u32 spins = 0;
    while (__hip_atomic_load(&ctl->seg_arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
      __builtin_amdgcn_s_sleep(1);
      if ((++spins & 1023u) == 0 && past_deadline(deadline)) {   // a block left on a time-out
        atomicOr(&ctl->status, MCE_E_TIMEOUT);
        res = PEEL_TIMEOUT;
        break;
      }
    }
    for (int i = 0; i < 3; i++) {
      pst<SA>(&ctl->fsize[i], 0);
      pst<SA>(&ctl->bsize[i], 0);
      pst<SA>(&ctl->bedge[i], 0);
    }
    pst<SA>(&ctl->asize[st.cur ^ 1], 0);
    pst<SA>(&ctl->asum[st.cur ^ 1], 0);
    pst<SA>(&ctl->min_deg[st.cur ^ 1], 0x7FFFFFFF);
    pst<SA>(&ctl->tmax[st.cur ^ 1], 0);
    __hip_atomic_store(&ctl->tsum[st.cur ^ 1], 0ull, __ATOMIC_RELAXED, SA);
    pst<SA>(&ctl->seg_state[0], res);
    pst<SA>(&ctl->seg_state[1], st.cur);
    pst<SA>(&ctl->seg_state[2], st.nf);
    pst<SA>(&ctl->seg_state[3], st.nb);
    pst<SA>(&ctl->seg_state[4], st.k);
    pst<SA>(&ctl->seg_state[5], st.r);
    pst<SA>(&ctl->seg_state[6], st.na);
    pst<SA>(&ctl->seg_state[7], st.level_known ? 1 : 0);
    pst<SA>(&ctl->seg_state[8], st.ph);
    pst<SA>(&ctl->seg_state[9], st.fe);
    pst<SA>(&ctl->seg_state[10], st.ae);
    wait_stores_complete();
    __hip_atomic_store(&ctl->seg_gen, st.seg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_res = res;
  }
  __syncthreads();
  return s_res;
}

// The other blocks while block 0 runs a segment: arrive, wait for its
// hand-back and take over its state. Returns what block 0 handed back
// (PEEL_TO_GRID: go on with the grid).
__device__ __forceinline__ int peel_wait(MceCtl* ctl, PeelState& st, u64 deadline) {
  __shared__ int s_late;
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(&ctl->seg_arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    u32 spins = 0;
    s_late = 0;
    while (__hip_atomic_load(&ctl->seg_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < st.seg) {
      __builtin_amdgcn_s_sleep(2);
      if ((++spins & 1023u) == 0 && past_deadline(deadline)) {
        atomicOr(&ctl->status, MCE_E_TIMEOUT);
        s_late = 1;
        break;
      }
    }
  }
  __syncthreads();
  if (s_late) return PEEL_TIMEOUT;
  const int res = pld<SA>(&ctl->seg_state[0]);
  st.cur = pld<SA>(&ctl->seg_state[1]);
  st.nf = pld<SA>(&ctl->seg_state[2]);
  st.nb = pld<SA>(&ctl->seg_state[3]);
  st.k = pld<SA>(&ctl->seg_state[4]);
  st.r = pld<SA>(&ctl->seg_state[5]);
  st.na = pld<SA>(&ctl->seg_state[6]);
  st.level_known = pld<SA>(&ctl->seg_state[7]) != 0;
  st.ph = pld<SA>(&ctl->seg_state[8]);
  st.fe = pld<SA>(&ctl->seg_state[9]);
  st.ae = pld<SA>(&ctl->seg_state[10]);
  return res;
}

// ------------------------------------------------------------------ the peel's tail
// Late in the peel few vertices remain, their rows still hold every removed
// neighbour, and the rounds left are many and small: each costs the grid a
// barrier and a few device-scope round trips. Once a level pass finds at most
// PEEL_TT vertices left (peel_rounds returns PEEL_TO_TAIL), every block writes
// the residual graph once, in local ids (a vertex's position in the remaining
// list), keeping only live entries, and block 0 finishes alone with the
// degrees in its LDS: a round is then one load of the frontier's rows and LDS
// atomics, with no grid barrier.
//
// peel_tail_build, every block. L = the remaining list (na entries).
//   a. block b takes L[bC, (b+1)C): rnd[v] = -2 - i marks v present with local
//      id i (any negative rnd still reads as present, and rnd is written again
//      when v leaves), the block-local prefix of the rows' sizes (tail_budget)
//      into tcrow[], the block's total into front1[b], the rows longer than
//      PEEL_TLONG into bfront0;
//   b. tcrow[] += the totals of the blocks before; tcrow[na] = all of them; the
//      long rows' write cursors (bfront1[i]) start at their row starts;
//   c. rows of at most PEEL_TLONG entries: one wavefront each, live entries in
//      CSR order, then 0xFFFF up to the row end; longer rows: PEEL_TSPAN-entry
//      spans dealt to every wavefront, each reserving its live entries rounded
//      up to 8 with an atomic on the row's cursor (the order of a row's
//      entries does not matter) and padding them;
//   d. the long rows' unreserved ends are padded.
// A vertex's degree is exactly its live entries (every removed neighbour took
// one). A row that would take more than its size sets MCE_E_PROTO instead of
// writing past it; so does a short row that ends with another count.
__device__ __forceinline__ int peel_tail_build(const PeelArgs& A, PeelState& st) {
  __shared__ long long s_bc[PEEL_THREADS / MCE_WAVE + 1];
  __shared__ long long s_off;
  const int lane = lane_id();
  const int na = st.na;
  const int* L = A.alive(st.cur);
  const int* __restrict__ rp = A.rp;
  const int* __restrict__ ci = A.ci;
  int* bsum = A.front1;      // per-block totals (int: at most tcap <= INT_MAX in all)
  int* longl = A.bfront0;    // local ids of the long rows
  int* cursor = A.bfront1;   // their write cursors, by local id
  int* livec = A.alive(st.cur ^ 1);   // and their live entries (the other remaining list is free)
  int* crow = A.tcrow;
  unsigned short* tcol = A.tcol;
  MceCtl* ctl = A.ctl;
  const int nblk = gridDim.x;
  const int C = (na + nblk - 1) / nblk;
  const int lo = min(na, (int)blockIdx.x * C), hi = min(na, lo + C);
  const int bw = threadIdx.x / MCE_WAVE, nbw = blockDim.x / MCE_WAVE;
  // a. local ids, block-local prefix of the row sizes, long rows
  long long run = 0;
  for (int base = lo; base < hi; base += PEEL_THREADS) {   // uniform in the block
    const int i = base + (int)threadIdx.x;
    long long sz = 0;
    bool lg = false;
    if (i < hi) {
      const int v = pld<SA>(&L[i]);
      const int d = pld<SA>(&A.deg[v]);
      const int len = rp[v + 1] - rp[v];
      sz = tail_budget(d, len);
      lg = len > PEEL_TLONG;
      pst<SA>(&A.rnd[v], -2 - i);
      if (A.snap) A.snap[v] = 1;
    }
    long long incl = sz;
#pragma unroll
    for (int o = 1; o < MCE_WAVE; o <<= 1) {
      const long long t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == MCE_WAVE - 1) s_bc[bw] = incl;
    const u64 lm = ballot(lg);
    int lpos = 0;
    if (lm && lane == 0) lpos = padd<SA>(&ctl->tlong, __popcll(lm));
    lpos = read_lane(lpos, 0);
    if (lg) pst<SA>(&longl[lpos + mbcnt(lm)], i);
    __syncthreads();
    if (threadIdx.x == 0) {
      long long r2 = 0;
      for (int w = 0; w < nbw; w++) {
        const long long c = s_bc[w];
        s_bc[w] = r2;
        r2 += c;
      }
      s_bc[nbw] = r2;
    }
    __syncthreads();
    if (i < hi) pst<SA>(&crow[i], (int)(run + s_bc[bw] + incl - sz));
    run += s_bc[nbw];
    __syncthreads();   // s_bc is filled again for the next piece
  }
  if (threadIdx.x == 0) pst<SA>(&bsum[blockIdx.x], (int)run);
  grid_sync(ctl, A.deadline, st.epoch);
  if (ld_relaxed(&ctl->status) & MCE_E_TIMEOUT) return PEEL_TIMEOUT;
  // b. the blocks' offsets
  if (bw == 0) {
    long long acc = 0, all = 0;
    for (int j = lane; j < nblk; j += MCE_WAVE) {
      const long long t = pld<SA>(&bsum[j]);
      all += t;
      if (j < (int)blockIdx.x) acc += t;
    }
    acc = (long long)wave_sum_u64((u64)acc);
    all = (long long)wave_sum_u64((u64)all);
    if (lane == 0) {
      s_off = acc;
      if (blockIdx.x == 0) pst<SA>(&crow[na], (int)all);
    }
  }
  __syncthreads();
  for (int i = lo + (int)threadIdx.x; i < hi; i += PEEL_THREADS) {
    const int c = pld<SA>(&crow[i]) + (int)s_off;
    pst<SA>(&crow[i], c);
    pst<SA>(&cursor[i], c);
    pst<SA>(&livec[i], 0);
  }
  grid_sync(ctl, A.deadline, st.epoch);
  if (ld_relaxed(&ctl->status) & MCE_E_TIMEOUT) return PEEL_TIMEOUT;
  // c. the live entries. Every rnd written so far went to memory with
  // agent-scope stores, and the barrier above orders them: with this XCD's L2
  // invalidated once, plain loads read them (-2 - local id: present).
  if (threadIdx.x == 0) fence_acquire_agent();
  __syncthreads();
  const int gw = (int)blockIdx.x * nbw + bw, ngw = nblk * nbw;
  u32 bad = 0;
  for (int i = gw; i < na; i += ngw) {
    const int v = pld<SA>(&L[i]);
    const int a = rp[v], b = rp[v + 1];
    if (b - a > PEEL_TLONG) continue;
    const int start = pld<SA>(&crow[i]);
    const int end = pld<SA>(&crow[i + 1]);
    const int d = pld<SA>(&A.deg[v]);
    int out = start;
    for (int e0 = a; e0 < b; e0 += PEEL_TSPAN) {
      int x[PEEL_TPER];
#pragma unroll
      for (int q = 0; q < PEEL_TPER; q++) {
        const int e = e0 + q * MCE_WAVE + lane;
        x[q] = e < b ? ci[e] : -1;
      }
#pragma unroll
      for (int q = 0; q < PEEL_TPER; q++) x[q] = x[q] >= 0 ? A.rnd[x[q]] : 0;
#pragma unroll
      for (int q = 0; q < PEEL_TPER; q++) {
        const bool live = x[q] <= -2;
        const u64 m = ballot(live);
        const int pos = out + mbcnt(m);
        if (live) {
          if (pos < end) tcol[pos] = (unsigned short)(-2 - x[q]);
          else bad = 1;
        }
        out += __popcll(m);
      }
    }
    if (out - start != d) bad = 1;
    for (int p = out + lane; p < end; p += MCE_WAVE) tcol[p] = (unsigned short)0xFFFFu;
  }
  const int nlong = pld<SA>(&ctl->tlong);
  for (int j0 = 0; j0 < nlong; j0 += MCE_WAVE) {
    const int jl = j0 + lane;
    const int il = jl < nlong ? pld<SA>(&longl[jl]) : 0;
    const int vl = jl < nlong ? pld<SA>(&L[il]) : 0;
    const int al = jl < nlong ? rp[vl] : 0, bl = jl < nlong ? rp[vl + 1] : 0;
    const int endl = jl < nlong ? pld<SA>(&crow[il + 1]) : 0;
    const int cnt = min(MCE_WAVE, nlong - j0);
    for (int t = 0; t < cnt; t++) {
      const int j = j0 + t;
      const int i = read_lane(il, t), a = read_lane(al, t), b = read_lane(bl, t), end = read_lane(endl, t);
      const int nsp = (b - a + PEEL_TSPAN - 1) / PEEL_TSPAN;
      for (int c = (gw - j % ngw + ngw) % ngw; c < nsp; c += ngw) {
        const int e0 = a + c * PEEL_TSPAN;
        int x[PEEL_TPER];
#pragma unroll
        for (int q = 0; q < PEEL_TPER; q++) {
          const int e = e0 + q * MCE_WAVE + lane;
          x[q] = e < b ? ci[e] : -1;
        }
#pragma unroll
        for (int q = 0; q < PEEL_TPER; q++) x[q] = x[q] >= 0 ? A.rnd[x[q]] : 0;
        int tot = 0;
#pragma unroll
        for (int q = 0; q < PEEL_TPER; q++) tot += __popcll(ballot(x[q] <= -2));
        const int sz = (tot + 7) & ~7;
        int base = 0;
        if (lane == 0 && sz) {
          base = padd<SA>(&cursor[i], sz);
          padd<SA>(&livec[i], tot);
        }
        base = read_lane(base, 0);
        if (sz && base + sz > end) {
          bad = 1;
          continue;
        }
        int out = base;
#pragma unroll
        for (int q = 0; q < PEEL_TPER; q++) {
          const bool live = x[q] <= -2;
          const u64 m = ballot(live);
          if (live) tcol[out + mbcnt(m)] = (unsigned short)(-2 - x[q]);
          out += __popcll(m);
        }
        if (lane < sz - tot) tcol[out + lane] = (unsigned short)0xFFFFu;
      }
    }
  }
  if (wave_or_u32(bad) && lane == 0) atomicOr(&ctl->status, MCE_E_PROTO);
  grid_sync(ctl, A.deadline, st.epoch);
  if (ld_relaxed(&ctl->status) & (MCE_E_TIMEOUT | MCE_E_PROTO)) return PEEL_TIMEOUT;
  // d. the long rows' ends past their last span; their live entries counted
  for (int j = gw; j < nlong; j += ngw) {
    const int i = pld<SA>(&longl[j]);
    const int c = pld<SA>(&cursor[i]);
    const int end = pld<SA>(&crow[i + 1]);
    for (int p = c + lane; p < end; p += MCE_WAVE) tcol[p] = (unsigned short)0xFFFFu;
    if (pld<SA>(&livec[i]) != pld<SA>(&A.deg[pld<SA>(&L[i])])) bad = 1;
  }
  if (wave_or_u32(bad) && lane == 0) atomicOr(&ctl->status, MCE_E_PROTO);
  // the rows were written with plain stores: out of this XCD's L2 before the
  // barrier (one write-back per block, after all of its waves' stores)
  wait_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) fence_release_agent();
  grid_sync(ctl, A.deadline, st.epoch);
  if (ld_relaxed(&ctl->status) & (MCE_E_TIMEOUT | MCE_E_PROTO)) return PEEL_TIMEOUT;
  return PEEL_TO_TAIL;
}

// Appends local id u of the lanes with `in` set to a tail frontier list: the
// LDS list holds PEEL_TFCAP entries, more go to the global list `ov`. Whole wave.
__device__ __forceinline__ void tail_push(bool in, int u, int* cnt, unsigned short* lst, int* ov) {
  const u64 m = ballot(in);
  if (!m) return;
  int pos = 0;
  if (lane_id() == 0) pos = atomicAdd(cnt, __popcll(m));
  pos = read_lane(pos, 0) + mbcnt(m);
  if (in) {
    if (pos < PEEL_TFCAP) lst[pos] = (unsigned short)u;
    else ov[pos - PEEL_TFCAP] = u;
  }
}

// One group of up to 64 frontier entries (lane t holds entry t: its row
// [a, b) in tcol, a multiple of 8 entries long; incl = the lanes' inclusive
// prefix of their rows' 8-entry chunks, C = all of them). The group's chunks
// are taken 64 at a time (a step: lane l takes chunk 64 s + l, whichever row
// it falls in, found by a binary search over the lanes' prefix); this wave
// takes steps sfirst, sfirst + sstep, ..., PEEL_TQ at a time (that many
// 16-byte loads per lane in flight), and takes one degree from every neighbour
// in them. A
// load's 8 decrements are issued before any returned value is read, and the
// joiners are appended only when the wave has any. Whole wave.
__device__ __forceinline__ void tail_chunks(int a, int incl, int C, int sfirst, int sstep, int na, int k, u32* deg,
                                            const unsigned short* __restrict__ tcol, int* cnt, unsigned short* nl,
                                            int* nov) {
  const int lane = lane_id();
  const int nsteps = (C + MCE_WAVE - 1) / MCE_WAVE;
  for (int s0 = sfirst; s0 < nsteps; s0 += PEEL_TQ * sstep) {
    uint4 w[PEEL_TQ];
#pragma unroll
    for (int q = 0; q < PEEL_TQ; q++) {
      const int c = (s0 + q * sstep) * MCE_WAVE + lane;
      w[q] = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);   // padding: no vertex
      if (s0 + q * sstep < nsteps) {
        // t = the lanes whose prefix is <= c: chunk c lies in lane t's row
        int t = 0;
#pragma unroll
        for (int step = 32; step > 0; step >>= 1) {
          const int v = __shfl(incl, t + step - 1);
          if (v <= c) t += step;
        }
        // (every lane takes part in each shuffle: a lane that sits one out
        // would read 0 from the lanes that do)
        const int tt = min(t, MCE_WAVE - 1);
        const int at = __shfl(a, tt);
        const int pre = __shfl(incl, max(tt - 1, 0));
        const int before = tt > 0 ? pre : 0;   // chunks of the rows before lane tt's
        if (c < C) w[q] = *reinterpret_cast<const uint4*>(tcol + at + (c - before) * 8);
      }
    }
    u32 jm = 0;
#pragma unroll
    for (int q = 0; q < PEEL_TQ; q++) {
      u32 old[8];
#pragma unroll
      for (int h = 0; h < 8; h++) {
        const u32 word = (h >> 1) == 0 ? w[q].x : (h >> 1) == 1 ? w[q].y : (h >> 1) == 2 ? w[q].z : w[q].w;
        const u32 u = (word >> ((h & 1) * 16)) & 0xFFFFu;
        old[h] = 0u;
        if ((int)u < na) old[h] = atomicSub(&deg[u >> 1], 1u << ((u & 1u) * 16u));
      }
#pragma unroll
      for (int h = 0; h < 8; h++) {
        const u32 word = (h >> 1) == 0 ? w[q].x : (h >> 1) == 1 ? w[q].y : (h >> 1) == 2 ? w[q].z : w[q].w;
        const u32 u = (word >> ((h & 1) * 16)) & 0xFFFFu;
        const u32 sh = (u & 1u) * 16u;
        if ((int)u < na && ((old[h] >> sh) & 0xFFFFu) == (u32)(k + 1)) {
          atomicOr(&deg[u >> 1], 0x8000u << sh);
          jm |= 1u << (q * 8 + h);
        }
      }
    }
    if (ballot(jm != 0u)) {
#pragma unroll
      for (int q = 0; q < PEEL_TQ; q++) {
#pragma unroll
        for (int h = 0; h < 8; h++) {
          const u32 word = (h >> 1) == 0 ? w[q].x : (h >> 1) == 1 ? w[q].y : (h >> 1) == 2 ? w[q].z : w[q].w;
          tail_push(((jm >> (q * 8 + h)) & 1u) != 0u, (int)((word >> ((h & 1) * 16)) & 0xFFFFu), cnt, nl, nov);
        }
      }
    }
  }
}

// Block 0 alone on the compacted residual graph, from the level peel_rounds
// ended at: the same rule (a level's first round is every remaining vertex of
// degree <= k; a round removes its frontier and a neighbour whose degree falls
// from k + 1 to k joins the next; when a round removes nothing, k rises to the
// smallest remaining degree). Degrees are packed 16-bit fields in LDS, two a
// word. A vertex's field gets bit 15 when it joins a frontier; it then takes
// exactly as many more decrements as neighbours of its that had not left when
// it was counted, so no field ever borrows from its neighbour in the word, and
// a field with bit 15 never reads k + 1 again. A round's rows are read in
// steps of 64 chunks of 8 entries (one 16-byte load per lane, see tail_chunks).
// A frontier of at most 64 entries has its steps dealt over all of the block's
// waves; a larger one is cut into one slice per wave, each taken 64 entries at
// a time (the next 64 entries' rows are loaded while a group's steps are
// taken). Rounds and core numbers are written through the remaining list.
__device__ __forceinline__ int peel_tail_rounds(const PeelArgs& A, PeelState& st, bool timer) {
  // [0..2] frontier sizes (rotating), [4] smallest field, [5] vertices of the tentative
  // level, [6] stop; s_wt: the waves' shares of a level's first round
  __shared__ int s_t[8];
  __shared__ int s_wt[PEEL_THREADS / MCE_WAVE + 1];
  const int lane = lane_id();
  const int bw = threadIdx.x / MCE_WAVE, nbw = blockDim.x / MCE_WAVE;
  const int na = st.na;
  const int nw = (na + 1) / 2;
  const int* L = A.alive(st.cur);
  const int* __restrict__ crow = A.tcrow;
  const unsigned short* __restrict__ tcol = A.tcol;
  u32* deg = A.pool;
  unsigned short* fl0 = (unsigned short*)(A.pool + (PEEL_TT + 1) / 2);
  unsigned short* fl1 = fl0 + PEEL_TFCAP;
  for (int w = threadIdx.x; w < nw; w += blockDim.x) {
    const u32 d0 = (u32)A.deg[L[2 * w]];
    const u32 d1 = 2 * w + 1 < na ? (u32)A.deg[L[2 * w + 1]] : 0x8000u;   // padding: gone already
    deg[w] = d0 | (d1 << 16);
  }
  if (threadIdx.x < 8) s_t[threadIdx.x] = 0;
  int k = st.k, r = st.r, cur = 0, nf = 0, slot = 0, rot = 0;
  bool entry = true;   // the level peel_rounds found: k is already that level
  __syncthreads();
  for (;;) {
    if (nf == 0) {
      // ---- a new level. Every remaining vertex has degree > k (>= k on
      // entry): the level is kt = k + 1 (k on entry) when some vertex has
      // that degree, else the smallest degree. Pass 1 finds the smallest field
      // (a removed vertex's is at least 0x8000, so it is the smallest degree
      // while any vertex remains) and counts the fields <= kt (all of them
      // remaining vertices' degrees); pass 2 collects the level's first round,
      // each thread's share placed by a block-wide scan. Both passes are
      // issue-bound (two fields a word): a few instructions a word.
      const int kdone = k;
      const int kt = entry ? k : k + 1;
      entry = false;
      if (threadIdx.x == 0) {
        s_t[(slot + 2) % 3] = 0;
        s_t[4] = 0x7FFFFFFF;
        s_t[5] = 0;
      }
      __syncthreads();
      u32 mn = 0xFFFFu;
      int le = 0;
      u32 wm = 0;   // bit j: word threadIdx.x + j * PEEL_THREADS holds some of them (nw <= 32 * PEEL_THREADS)
      for (int j0 = 0; j0 * PEEL_THREADS < nw; j0 += 4) {
        u32 x[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int w = (j0 + q) * PEEL_THREADS + (int)threadIdx.x;
          x[q] = w < nw ? deg[w] : 0xFFFFFFFFu;
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const u32 f0 = x[q] & 0xFFFFu, f1 = x[q] >> 16;
          mn = min(mn, min(f0, f1));
          const int c2 = ((int)f0 <= kt) + ((int)f1 <= kt);
          le += c2;
          wm |= c2 ? 1u << (j0 + q) : 0u;
        }
      }
      const int wle = (int)wave_sum_u32((u32)le);
      const int wmn = wave_min_i32_nonneg((int)mn);
      if (lane == 0) {
        if (wle) atomicAdd(&s_t[5], wle);
        atomicMin(&s_t[4], wmn);
      }
      __syncthreads();
      if (s_t[4] >= 0x8000) {   // every field marked: no vertex remains
        PEEL_MARK(tl);
        st.k = kdone;
        st.r = r;
        st.na = 0;
        return PEEL_DONE;
      }
      k = s_t[5] > 0 ? kt : s_t[4];
      int c = le;
      if (s_t[5] == 0) {   // a jump: this thread's vertices of the smallest degree
        c = 0;
        wm = 0;
        for (int j = 0; j * PEEL_THREADS < nw; j++) {
          const int w = j * PEEL_THREADS + (int)threadIdx.x;
          const u32 x = w < nw ? deg[w] : 0xFFFFFFFFu;
          const int c2 = ((int)(x & 0xFFFFu) == k) + ((int)(x >> 16) == k);
          c += c2;
          wm |= c2 ? 1u << j : 0u;
        }
      }
      // pass 2: this thread's vertices of degree <= k, marked, at its place in the list
      int incl = c;
#pragma unroll
      for (int o = 1; o < MCE_WAVE; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      if (lane == MCE_WAVE - 1) s_wt[bw] = incl;
      __syncthreads();
      if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < nbw; i++) {
          const int t = s_wt[i];
          s_wt[i] = run;
          run += t;
        }
        s_wt[nbw] = run;
      }
      __syncthreads();
      {
        unsigned short* fl = cur ? fl1 : fl0;
        int* ov = cur ? A.front1 : A.front0;
        int pos = s_wt[bw] + incl - c;
        while (wm) {
          const int w = __builtin_ctz(wm) * PEEL_THREADS + (int)threadIdx.x;
          wm &= wm - 1u;
          u32 x = deg[w];
          const u32 f0 = x & 0xFFFFu, f1 = x >> 16;
          const bool in0 = (int)f0 <= k, in1 = (int)f1 <= k;   // k < 0x8000: remaining vertices only
          if (in0) {
            x |= 0x8000u;
            if (pos < PEEL_TFCAP) fl[pos] = (unsigned short)(2 * w);
            else ov[pos - PEEL_TFCAP] = 2 * w;
            pos++;
          }
          if (in1) {
            x |= 0x80000000u;
            if (pos < PEEL_TFCAP) fl[pos] = (unsigned short)(2 * w + 1);
            else ov[pos - PEEL_TFCAP] = 2 * w + 1;
            pos++;
          }
          if (in0 || in1) deg[w] = x;
        }
      }
      nf = s_wt[nbw];
      slot = (slot + 1) % 3;
      __syncthreads();
      PEEL_MARK(tl);
    }
    // ---- round r: remove the frontier (list cur), take one degree from each neighbour
    if ((r & 63) == 0) {
      if (threadIdx.x == 0) s_t[6] = past_deadline(A.deadline) ? 1 : 0;
      __syncthreads();
      if (s_t[6]) {
        if (threadIdx.x == 0) atomicOr(&A.ctl->status, MCE_E_TIMEOUT);
        return PEEL_TIMEOUT;
      }
    }
    const int p1 = (slot + 1) % 3;
    if (threadIdx.x == 0) s_t[(slot + 2) % 3] = 0;
    const unsigned short* fl = cur ? fl1 : fl0;
    const int* ov = cur ? A.front1 : A.front0;
    unsigned short* nl = cur ? fl0 : fl1;
    int* nov = cur ? A.front0 : A.front1;
    // this wave's entries: all of a frontier of at most 64 (pieces shared by
    // all waves), else a slice of about nf / nbw
    const bool shared = nf <= MCE_WAVE;
    const int lo = shared ? 0 : (int)(((long long)nf * bw) / nbw);
    const int hi = shared ? nf : (int)(((long long)nf * (bw + 1)) / nbw);
    int li = -1, a = 0, b = 0;
    if (lo + lane < hi) {
      const int j = lo + lane;
      li = j < PEEL_TFCAP ? (int)fl[j] : ov[j - PEEL_TFCAP];
      a = crow[li];
      b = crow[li + 1];
    }
    for (int g0 = lo; g0 < hi; g0 += MCE_WAVE) {
      // the next group's rows are in flight while this group's pieces are taken
      int lin = -1, an = 0, bn = 0;
      if (g0 + MCE_WAVE + lane < hi) {
        const int j = g0 + MCE_WAVE + lane;
        lin = j < PEEL_TFCAP ? (int)fl[j] : ov[j - PEEL_TFCAP];
        an = crow[lin];
        bn = crow[lin + 1];
      }
      // the group's vertices leave in round r (one wave writes them)
      if (li >= 0 && (!shared || bw == r % nbw)) {
        const int v = L[li];
        A.rnd[v] = r;
        A.core[v] = k;
      }
      int incl = (b - a) >> 3;   // the row's 8-entry chunks
#pragma unroll
      for (int o = 1; o < MCE_WAVE; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const int C = read_lane(incl, MCE_WAVE - 1);
      if (shared) {
        // step s goes to wave (s + rot) mod nbw; rot moves on, so that rounds
        // of few steps do not all start on the same waves
        const int S = (C + MCE_WAVE - 1) / MCE_WAVE;
        tail_chunks(a, incl, C, ((bw - rot) % nbw + nbw) % nbw, nbw, na, k, deg, tcol, &s_t[p1], nl, nov);
        rot = (rot + S) % nbw;
      } else {
        tail_chunks(a, incl, C, 0, 1, na, k, deg, tcol, &s_t[p1], nl, nov);
      }
      li = lin;
      a = an;
      b = bn;
    }
    PEEL_MARK(tr);
    __syncthreads();
    nf = s_t[p1];
    slot = p1;
    cur ^= 1;
    r++;
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
// again (that needs a fall from k+1). Launched cooperatively; one block for
// small graphs. Most rounds of a large sparse graph remove a handful of
// vertices, and a grid barrier costs more than their work: a round of at most
// PEEL_TINY vertices whose big rows hold at most PEEL_SEG_EDGES edges is run by
// block 0 alone (peel_seg), with its frontier in LDS, while the other blocks
// wait for it to hand back a larger round or a level pass. Once at most
// PEEL_SOLO vertices with at most PEEL_SOLO_EDGES edges in their rows remain,
// block 0 finishes alone at workgroup scope and the other blocks leave.
__global__ __launch_bounds__(PEEL_THREADS) void k_peel(int n, const int* __restrict__ rp,
                                                        const int* __restrict__ ci, int* deg, int* rnd, int* core,
                                                        int* alive0, int* alive1, int* front0, int* front1,
                                                        int* bfront0, int* bfront1, MceCtl* ctl, u64 budget,
                                                        unsigned short* tcol, long long tcap, int* tcrow,
                                                        int split, unsigned char* snap) {
  __shared__ int s_cnt[12];
  __shared__ int4 s_fr[2 * PEEL_TINY + 1];
  // One LDS pool, used one of two ways in a launch:
  //  - a graph of at most PEEL_LDS_N vertices peeled by one block keeps
  //    degrees, rounds and the list and frontier counters in LDS (a copy of the
  //    control block): the peel's generic loads, stores and atomics then go to
  //    LDS instead of the L2, and a round's barrier waits on no global store
  //    (the rounds and any status bit are copied out at the end);
  //  - block 0 of a grid peel, in its tail: packed degrees and frontier lists.
  __shared__ __align__(128) u32 s_pool[PEEL_TPOOL];
  static_assert(2 * PEEL_LDS_N + (sizeof(MceCtl) + 3) / 4 <= PEEL_TPOOL, "the small-graph state fits the pool");
  static_assert(alignof(MceCtl) <= 128 && (2 * PEEL_LDS_N * 4) % alignof(MceCtl) == 0,
                "the control block's copy is aligned in the pool");
  int* s_deg = (int*)s_pool;
  int* s_rnd = s_deg + PEEL_LDS_N;
  MceCtl* s_ctl = (MceCtl*)(s_pool + 2 * PEEL_LDS_N);
  if (ld_relaxed(&ctl->status) != 0) return;   // rejected input: nothing to order
  const u64 t0 = wall_clock64();
  const bool lds = gridDim.x == 1 && n <= PEEL_LDS_N;
  MceCtl* pc = lds ? s_ctl : ctl;   // the peel's counters
  if (lds) {
    for (int i = threadIdx.x; i < (int)(sizeof(MceCtl) / sizeof(u32)); i += blockDim.x) ((u32*)s_ctl)[i] = 0u;
    __syncthreads();
  }
  PeelArgs A{n,      rp,     ci,      lds ? s_deg : deg, lds ? s_rnd : rnd, core,        alive0,
             alive1, front0, front1,  bfront0,           bfront1,           pc,          t0 + budget,
             s_cnt,  s_fr,   tcol,    gridDim.x > 1 ? tcap : 0LL,           tcrow,       s_pool,
             split ? snap : nullptr};
  const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
  const int gsize = gridDim.x * blockDim.x;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  // k starts below every degree: the first level is the smallest degree
  PeelState st{0, 0, 0, -1, 0, n, 0, 0, 0, 0, 0, false, 0u, 0u, 0, 0, 0, t0};

  for (int v = gtid; v < n; v += gsize) {
    pst<SA>(&A.deg[v], rp[v + 1] - rp[v]);
    pst<SA>(&A.rnd[v], -1);
    pst<SA>(&alive0[v], v);
  }
  if (gtid == 0) {
    st_relaxed64(&ctl->t_run, t0);
    pst<SA>(&pc->asize[0], n);
    pst<SA>(&pc->asize[1], 0);
    for (int i = 0; i < 3; i++) {
      pst<SA>(&pc->fsize[i], 0);
      pst<SA>(&pc->bsize[i], 0);
      pst<SA>(&pc->bedge[i], 0);
    }
    pst<SA>(&pc->asum[0], 0);
    pst<SA>(&pc->asum[1], 0);
    pst<SA>(&pc->min_deg[0], 0x7FFFFFFF);
    pst<SA>(&pc->min_deg[1], 0x7FFFFFFF);
    for (int i = 0; i < 2; i++) {
      pst<SA>(&pc->tmax[i], 0);
      __hip_atomic_store(&pc->tsum[i], 0ull, __ATOMIC_RELAXED, SA);
    }
    pst<SA>(&pc->tlong, 0);
  }
  grid_sync(ctl, A.deadline, st.epoch);

  const int bwave = threadIdx.x / MCE_WAVE, bwaves = blockDim.x / MCE_WAVE;
  int res;
  if (gridDim.x > 1) {
    for (;;) {
      res = peel_rounds<SA, PEEL_GRID>(A, st, gtid / MCE_WAVE, gsize / MCE_WAVE, timer);
      if (res == PEEL_TO_SEG) {
        st.seg++;
        if (blockIdx.x != 0) {
          res = peel_wait(ctl, st, A.deadline);
          if (res == PEEL_TO_GRID) continue;
          return;   // block 0 finishes the peel (or it timed out)
        }
        res = peel_seg(A, st, bwave, bwaves, timer);
        // hand back: a larger round or a level pass for the grid, or leave
        res = peel_hand_back(ctl, st, res, A.deadline);
        if (res == PEEL_TO_GRID) continue;
      }
      if (res == PEEL_TO_TAIL) {
        // every block writes the compacted residual graph; block 0 finishes on it
        res = peel_tail_build(A, st);
        if (blockIdx.x != 0) return;
        if (res == PEEL_TO_TAIL) {
          if (split) {
            // the tail is k_peel_tail's, a launch of its own: hand over the
            // state (this launch's end makes all of its writes visible to the
            // launches that follow it)
            if (threadIdx.x == 0) {
              ctl->tail_st[0] = st.k;
              ctl->tail_st[1] = st.r;
              ctl->tail_st[2] = st.na;
              ctl->tail_st[3] = st.cur;
              ctl->tail_ticks[0] = st.tb;
              ctl->tail_ticks[1] = st.tl;
              ctl->tail_ticks[2] = st.tr;
              ctl->tail_r0 = st.r;
              ctl->tail_go = 1;
            }
            return;
          }
          fence_acquire_agent();
          res = peel_tail_rounds(A, st, timer);
        }
        break;
      }
      if (res == PEEL_TO_ALONE) {
        if (blockIdx.x != 0) return;
        // block 0 goes on alone: drop any stale copy its XCD's caches may hold
        // of what the other blocks wrote
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        res = peel_rounds<SW, PEEL_ALONE>(A, st, bwave, bwaves, timer);
      }
      break;
    }
  } else {
    res = peel_rounds<SW, PEEL_ALONE>(A, st, bwave, bwaves, timer);
  }
  if (lds && threadIdx.x == 0 && s_ctl->status) atomicOr(&ctl->status, s_ctl->status);
  if (res < 0) return;
  if (lds) {
    __syncthreads();
    for (int v = threadIdx.x; v < n; v += blockDim.x) rnd[v] = s_rnd[v];
  }
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    ctl->rounds = st.r;
    ctl->degeneracy = max(st.k, 0);
    ctl->peel_ticks[0] = st.tb;
    ctl->peel_ticks[1] = st.tl;
    ctl->peel_ticks[2] = st.tr;
    ctl->peel_ticks[3] = wall_clock64() - t0;
  }
}

// The split peel's second launch: block 0's tail on the compacted residual
// graph (peel_tail_rounds), from the state the grid handed over. It runs as an
// ordinary one-block launch, so kernels on other streams can use the rest of
// the chip meanwhile (the subtrees of the vertices that have left already).
// Nothing to do when the grid peeled to the end or stopped.
__global__ __launch_bounds__(PEEL_THREADS) void k_peel_tail(int n, const int* __restrict__ rp,
                                                             const int* __restrict__ ci, int* deg, int* rnd,
                                                             int* core, int* alive0, int* alive1, int* front0,
                                                             int* front1, int* bfront0, int* bfront1, MceCtl* ctl,
                                                             u64 budget, unsigned short* tcol, long long tcap,
                                                             int* tcrow) {
  __shared__ int s_cnt[12];
  __shared__ int4 s_fr[2 * PEEL_TINY + 1];
  __shared__ __align__(128) u32 s_pool[PEEL_TPOOL];
  if (ctl->tail_go == 0) return;
  const u64 t0 = ctl->t_run;
  PeelArgs A{n,      rp,     ci,     deg,    rnd,   core, alive0, alive1, front0, front1,
             bfront0, bfront1, ctl,  t0 + budget, s_cnt, s_fr, tcol,   tcap,   tcrow,  s_pool, nullptr};
  const bool timer = threadIdx.x == 0;
  PeelState st{0, 0, 0, -1, 0, 0, 0, 0, 0, 0, 0, false, 0u, 0u, 0, 0, 0, 0};
  st.k = ctl->tail_st[0];
  st.r = ctl->tail_st[1];
  st.na = ctl->tail_st[2];
  st.cur = ctl->tail_st[3];
  st.tb = ctl->tail_ticks[0];
  st.tl = ctl->tail_ticks[1];
  st.tr = ctl->tail_ticks[2];
  st.tm = wall_clock64();
  const int res = peel_tail_rounds(A, st, timer);
  if (res < 0) return;
  if (threadIdx.x == 0) {
    ctl->rounds = st.r;
    ctl->degeneracy = max(st.k, 0);
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
// A block's sub-class tallies, in LDS: the waves add to them with LDS atomics
// and the block adds them to the control block once, at its end (same-address
// atomics in device memory serialise: one set per wave cost the orientation of
// a 500k-vertex graph about 0.5 ms).
struct TallyAcc {
  int count[MCE_NVAR][MCE_NSUB];
  int maxp[MCE_NVAR][MCE_NSUB];
  int maxx[MCE_NVAR][MCE_NSUB];
  int maxr[MCE_NVAR][MCE_NSUB];
  u64 words[MCE_NVAR][MCE_NSUB];
};

// Clears the block's tallies and reads whether the run still goes on (status
// clear), one read for the whole block so that every thread takes the same way
// (the kernels that tally end with a block barrier). Whole block.
__device__ __forceinline__ bool tally_begin(TallyAcc& t, int* s_ok, MceCtl* ctl) {
  for (int i = threadIdx.x; i < MCE_NVAR * MCE_NSUB; i += blockDim.x) {
    (&t.count[0][0])[i] = 0;
    (&t.maxp[0][0])[i] = 0;
    (&t.maxx[0][0])[i] = 0;
    (&t.maxr[0][0])[i] = 0;
    (&t.words[0][0])[i] = 0ull;
  }
  if (threadIdx.x == 0) *s_ok = ld_relaxed(&ctl->status) == 0 ? 1 : 0;
  __syncthreads();
  return *s_ok != 0;
}

// Adds the block's tallies to the control block. Whole block.
__device__ __forceinline__ void tally_end(TallyAcc& t, MceCtl* ctl) {
  __syncthreads();
  for (int i = threadIdx.x; i < MCE_NVAR * MCE_NSUB; i += blockDim.x) {
    const int var = i / MCE_NSUB, sub = i % MCE_NSUB;
    if (t.count[var][sub] == 0) continue;
    atomicAdd(&ctl->sub_count[var][sub], t.count[var][sub]);
    atomicMax(&ctl->sub_maxp[var][sub], t.maxp[var][sub]);
    atomicMax(&ctl->sub_maxx[var][sub], t.maxx[var][sub]);
    atomicMax(&ctl->sub_maxr[var][sub], t.maxr[var][sub]);
    atomicAdd(&ctl->sub_words[var][sub], t.words[var][sub]);
  }
}

// Tallies a wave's roots (one per lane, `valid` set) per classification variant
// (subgraph mode, micro sub-class on or off) and sub-class: count, largest |P|,
// |X| and row count, heap words, into the block's tallies. Whole wave.
__device__ __forceinline__ void tally_roots(TallyAcc& acc, bool valid, int p, int x) {
  const int lane = lane_id();
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
        atomicAdd(&acc.count[var][s], __popcll(m));
        atomicMax(&acc.maxp[var][s], (int)mp);
        atomicMax(&acc.maxx[var][s], (int)mx);
        atomicMax(&acc.maxr[var][s], (int)mr);
        atomicAdd(&acc.words[var][s], words);
      }
    }
  }
}

#define ORIENT_LONG 128   // rows longer than this are counted by the whole wavefront
#define ORIENT_MUL 2654435761u   // a prime above every int32 root count

// Later (|P|) and earlier (|X|) neighbours of every root. With many roots one
// thread takes each root (a wavefront takes each long row in turn); with at most
// one root per wavefront of the grid (per_wave), each wavefront takes one root
// and its lanes share the row: a thread alone would walk the row one dependent
// pair of loads (entry, then its round) at a time. With the forward adjacency
// already counted (fdeg, every vertex a root) |P| is read, not counted.

__global__ __launch_bounds__(256) void k_orient(int n, const int* __restrict__ rp, const int* __restrict__ ci,
                                                 const int* __restrict__ rnd, const int* __restrict__ roots,
                                                 int nroots, int* pcount, int* xcount, MceCtl* ctl, u64* fwd,
                                                 const int* __restrict__ fdeg, int tally, int per_wave, u32 mul) {
  __shared__ TallyAcc s_tally;
  __shared__ int s_ok;
  if (!tally_begin(s_tally, &s_ok, ctl)) return;

  const int lane = lane_id();
  const int gsize = gridDim.x * blockDim.x;
  const int cnt = nroots;   // roots == NULL: the identity list 0..nroots-1
  u64 iso = 0, iso_hash = 0;
  int pmax = 0, xmax = 0, dmax = 0;
  u32 lim = 0;
  if (per_wave) {
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / MCE_WAVE;
    for (int i = wave; i < cnt; i += gsize / MCE_WAVE) {
      const int v = roots ? roots[i] : i;
      if (v < 0 || v >= n) {   // caller-supplied root out of range: flag it, touch nothing
        if (lane == 0) {
          lim |= 2u;
          pcount[i] = 0;
          xcount[i] = 0;
          if (fwd) fwd[i] = 0;
        }
        continue;
      }
      const int a = rp[v], b = rp[v + 1], rv = rnd[v];
      u32 c = 0;
      for (int e = a + lane; e < b; e += MCE_WAVE) {
        const int u = ci[e];
        c += order_after(rnd[u], u, rv, v) ? 1u : 0u;
      }
      const int p = (int)wave_sum_u32(c), x = (b - a) - p;
      if (lane == 0) {
        pcount[i] = p;
        xcount[i] = x;
        if (fwd) fwd[i] = (u64)p;
        if (b == a) {
          iso++;
          iso_hash += mce_clique_term(mce_vertex_term(v), 1);
        }
        pmax = max(pmax, p);
        xmax = max(xmax, x);
        dmax = max(dmax, b - a);
        if (tally && p > MCE_MAX_P) lim |= 1u;
      }
    }   // the tallies follow in k_tally (64 roots at a time: one root each would
        // cost a score of same-address atomics)
  } else {
    for (int base = blockIdx.x * blockDim.x; base < cnt; base += gsize) {
      // thread tid takes root tid * mul mod cnt (mul a prime above cnt: a
      // permutation), so that roots of neighbouring ids, such as the hubs of
      // a graph whose degrees fall with the id, fall to different wavefronts
      const int tid = base + threadIdx.x;
      const int i = tid < cnt ? (int)((u64)tid * mul % (u64)cnt) : tid;
      int p = 0, x = 0;
      bool valid = false;
      const int v = i < cnt ? (roots ? roots[i] : i) : 0;
      if (i < cnt && (v < 0 || v >= n)) {   // caller-supplied root out of range: flag it, touch nothing
        lim |= 2u;
        pcount[i] = 0;
        xcount[i] = 0;
      }
      // later neighbours: one thread per short row; the whole wavefront takes each
      // long row in turn (a hub row would keep one thread busy for its whole length)
      const bool inr = i < cnt && v >= 0 && v < n;
      int a = 0, b = 0, rv = 0;
      if (inr) {
        a = rp[v];
        b = rp[v + 1];
        rv = rnd[v];
      }
      const bool longrow = inr && !fdeg && b - a > ORIENT_LONG;
      if (inr && fdeg) {
        p = fdeg[v];
      } else if (inr && !longrow) {
        // four entries at a time: their loads, then their rounds' loads, overlap
        int e = a;
        for (; e + 4 <= b; e += 4) {
          int u[4], r[4];
#pragma unroll
          for (int z = 0; z < 4; z++) u[z] = ci[e + z];
#pragma unroll
          for (int z = 0; z < 4; z++) r[z] = rnd[u[z]];
#pragma unroll
          for (int z = 0; z < 4; z++) p += order_after(r[z], u[z], rv, v) ? 1 : 0;
        }
        for (; e < b; e++) {
          const int u = ci[e];
          p += order_after(rnd[u], u, rv, v) ? 1 : 0;
        }
      }
      for (u64 lm = ballot(longrow); lm; lm &= lm - 1ull) {
        const int t = __builtin_ctzll(lm);
        const int ta = read_lane(a, t), tb = read_lane(b, t), tv = read_lane(v, t), tr = read_lane(rv, t);
        u32 c = 0;
        for (int e = ta + lane; e < tb; e += MCE_WAVE) {
          const int u = ci[e];
          c += order_after(rnd[u], u, tr, tv) ? 1u : 0u;
        }
        c = wave_sum_u32(c);
        if (lane == t) p = (int)c;
      }
      if (inr) {
        x = (b - a) - p;
        pcount[i] = p;
        xcount[i] = x;
        if (fwd) fwd[i] = (u64)p;
        if (b == a) {
          iso++;
          iso_hash += mce_clique_term(mce_vertex_term(v), 1);
        }
        pmax = max(pmax, p);
        xmax = max(xmax, x);
        dmax = max(dmax, b - a);
        if (tally && p > MCE_MAX_P) lim |= 1u;
        valid = p > 0 && p <= MCE_MAX_P;
      } else if (i < cnt && fwd) {
        fwd[i] = 0;
      }
      if (tally) tally_roots(s_tally, valid, p, x);
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
  if (tally) tally_end(s_tally, ctl);
}

// Forward adjacency of every vertex (the oriented graph of section 2.4): the
// neighbours after v in the peel order, kept at the start of v's own CSR span
// (so no offsets need computing), and their number. Micro-table builds read
// these rows instead of whole CSR rows: every edge between two members of a
// subtree's P u X sits in the forward row of its earlier end, and a forward row
// is no longer than that end's core number, where a CSR row can be as long as
// the maximum degree. The readers look every entry up in a hash, so the order
// of a forward row is free, but both passes keep it in id order: rows of up
// to FWD_LONG entries are taken by one wavefront (a ballot keeps them in order);
// a longer row is only listed here, and k_forward_adj_long gives each one a
// whole block that takes 1,024 entries at a time (a hub's row, tens of
// thousands of entries on power-law graphs, kept one wavefront busy for
// milliseconds).
//
// With tctl (a split peel's control block): nothing is done unless the grid
// handed a tail over (the rows are then those of the hand-over order, rnd being
// its ranks, see k_search_rank).
#define FWD_LONG 1024

__global__ __launch_bounds__(256) void k_forward_adj(int n, const int* __restrict__ rp, const int* __restrict__ ci,
                                                      const int* __restrict__ rnd, int* __restrict__ fadj,
                                                      int* __restrict__ fdeg, int* __restrict__ flong, MceCtl* ctl,
                                                      const MceCtl* tctl) {
  if (tctl && !tctl->tail_go) return;
  // the block's long rows, listed in LDS and added to the list with one atomic
  // (one per row on the shared count took a 4M-vertex graph's ~20k hub rows
  // about 0.3 ms); a block with more than FWD_LCAP of them lists the rest
  // directly
  constexpr int FWD_LCAP = 256;
  __shared__ int s_long[FWD_LCAP];
  __shared__ int s_nl, s_base;
  if (threadIdx.x == 0) s_nl = 0;
  __syncthreads();
  const int lane = lane_id();
  const int nwaves = gridDim.x * (blockDim.x / MCE_WAVE);
  for (int v = blockIdx.x * (blockDim.x / MCE_WAVE) + threadIdx.x / MCE_WAVE; v < n; v += nwaves) {
    const int a = rp[v], b = rp[v + 1], rv = rnd[v];
    if (b - a > FWD_LONG) {
      if (lane == 0) {
        const int q = atomicAdd(&s_nl, 1);
        if (q < FWD_LCAP) s_long[q] = v;
        else flong[atomicAdd(&ctl->nlong, 1)] = v;
      }
      continue;
    }
    int k = 0;
    for (int base = a; base < b; base += MCE_WAVE) {
      const int e = base + lane;
      const int u = e < b ? ci[e] : 0;
      const bool later = e < b && order_after(rnd[u], u, rv, v);
      const u64 m = ballot(later);
      if (later) fadj[a + k + mbcnt(m)] = u;
      k += __popcll(m);
    }
    if (lane == 0) fdeg[v] = k;
  }
  __syncthreads();
  const int nl = min(s_nl, FWD_LCAP);
  if (threadIdx.x == 0) s_base = nl ? atomicAdd(&ctl->nlong, nl) : 0;
  __syncthreads();
  for (int i = threadIdx.x; i < nl; i += blockDim.x) flong[s_base + i] = s_long[i];
}

// The long rows listed by k_forward_adj, one block per row: each thread loads
// four entries (then their rounds) per step, and the block places the step's
// later entries in order (entry groups z, then wavefronts) behind the ones
// already placed.
__global__ __launch_bounds__(256) void k_forward_adj_long(const int* __restrict__ rp, const int* __restrict__ ci,
                                                           const int* __restrict__ rnd, int* __restrict__ fadj,
                                                           int* __restrict__ fdeg, const int* __restrict__ flong,
                                                           MceCtl* ctl, const MceCtl* tctl) {
  constexpr int NW = 256 / MCE_WAVE;
  __shared__ int s_cnt[4][NW];
  if (tctl && !tctl->tail_go) return;
  const int lane = lane_id(), wv = threadIdx.x / MCE_WAVE;
  const int nl = ld_relaxed(&ctl->nlong);
  for (int j = blockIdx.x; j < nl; j += gridDim.x) {
    const int v = flong[j];
    const int a = rp[v], b = rp[v + 1], rv = rnd[v];
    int k = 0;   // entries placed so far (the same in every thread)
    for (int base = a; base < b; base += 4 * 256) {
      int u[4];
      bool lat[4];
      u64 m[4];
#pragma unroll
      for (int z = 0; z < 4; z++) {
        const int e = base + z * 256 + (int)threadIdx.x;
        u[z] = e < b ? ci[e] : 0;
      }
#pragma unroll
      for (int z = 0; z < 4; z++) {
        const int e = base + z * 256 + (int)threadIdx.x;
        lat[z] = e < b && order_after(rnd[u[z]], u[z], rv, v);
      }
#pragma unroll
      for (int z = 0; z < 4; z++) {
        m[z] = ballot(lat[z]);
        if (lane == 0) s_cnt[z][wv] = __popcll(m[z]);
      }
      __syncthreads();
      int before = k, total = 0;
#pragma unroll
      for (int z = 0; z < 4; z++) {
        int off = before;
        for (int w = 0; w < NW; w++) {
          if (w < wv) off += s_cnt[z][w];
          total += s_cnt[z][w];
        }
        if (lat[z]) fadj[a + off + mbcnt(m[z])] = u[z];
        for (int w = 0; w < NW; w++) before += s_cnt[z][w];
      }
      k += total;
      __syncthreads();   // s_cnt is rewritten by the next step
    }
    if (threadIdx.x == 0) fdeg[v] = k;
  }
}

// The sub-class tallies of the roots that k_orient counted one wavefront per
// root: one thread per root, grouped per wavefront as in k_orient.
__global__ __launch_bounds__(256) void k_tally(int nroots, const int* __restrict__ pcount,
                                                const int* __restrict__ xcount, MceCtl* ctl) {
  __shared__ TallyAcc s_tally;
  __shared__ int s_ok;
  if (!tally_begin(s_tally, &s_ok, ctl)) return;
  const int gsize = gridDim.x * blockDim.x;
  for (int base = blockIdx.x * blockDim.x; base < nroots; base += gsize) {
    const int i = base + threadIdx.x;
    const int p = i < nroots ? pcount[i] : 0, x = i < nroots ? xcount[i] : 0;
    tally_roots(s_tally, p > 0 && p <= MCE_MAX_P, p, x);
  }
  tally_end(s_tally, ctl);
}

// A split peel's hand-over order, as ranks compared like rounds (rank, then
// id): a vertex gone before the tail keeps its round; a vertex still in the
// tail (snap 1) gets r0 + its degree in the remaining graph (deg, which the
// tail leaves as it was handed over), so it comes after every vertex gone and,
// among the tail's, by that degree, then id. Every maximal clique is reported
// once under any vertex order (the subtree of its first vertex, section 2.4);
// the degeneracy order is what bounds |P|, and the hand-over order keeps it
// where the peel left off. The round of a tail vertex is not read: the tail
// writes it meanwhile.
__global__ __launch_bounds__(256) void k_search_rank(int n, const int* __restrict__ rnd, const int* __restrict__ deg,
                                                     const unsigned char* __restrict__ snap, const MceCtl* tctl,
                                                     int* srank) {
  if (!tctl->tail_go) return;
  const int r0 = tctl->tail_r0;
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < n; v += gridDim.x * blockDim.x)
    srank[v] = snap[v] ? r0 + deg[v] : rnd[v];
}

// The roots of a split peel's hand-over order (every vertex gone before the
// tail by its round, then the tail's vertices by their degree in the remaining
// graph, then id: the order of the early forward adjacency, whose fdeg is |P|).
// Like k_orient's thread-per-root pass: |P| and |X| of every vertex into pcount /
// xcount, the sub-class tallies, the largest |P|, |X| and degree, the isolated
// vertices (maximal cliques of one) into `ctl` (a control block of its own),
// with the grid's hand-over facts copied there for the host: tail_go, tail_r0,
// and the level reached (a lower bound of the degeneracy) in `degeneracy`.
__global__ __launch_bounds__(256) void k_orient_handover(int n, const int* __restrict__ rp,
                                                         const int* __restrict__ fdeg, const MceCtl* tctl,
                                                         int* pcount, int* xcount, MceCtl* ctl) {
  __shared__ TallyAcc s_tally;
  __shared__ int s_ok;
  if (!tally_begin(s_tally, &s_ok, ctl)) return;
  const int go = tctl->tail_go;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ctl->tail_go = go;
    ctl->tail_r0 = go ? tctl->tail_r0 : -1;
    ctl->degeneracy = go ? tctl->tail_st[0] : 0;
    ctl->max_degree = tctl->max_degree;
  }
  if (!go) return;   // (a block-uniform exit: every thread read the same word)
  const int lane = lane_id();
  u64 iso = 0, iso_hash = 0;
  int pmax = 0, xmax = 0;
  u32 lim = 0;
  const int gsize = gridDim.x * blockDim.x;
  for (int base = blockIdx.x * blockDim.x; base < n; base += gsize) {
    const int v = base + threadIdx.x;
    int p = 0, x = 0;
    if (v < n) {
      p = fdeg[v];
      x = (rp[v + 1] - rp[v]) - p;
      pcount[v] = p;
      xcount[v] = x;
      if (p == 0 && x == 0) {
        iso++;
        iso_hash += mce_clique_term(mce_vertex_term(v), 1);
      }
      pmax = max(pmax, p);
      xmax = max(xmax, x);
      if (p > MCE_MAX_P) lim |= 1u;
    }
    tally_roots(s_tally, p > 0 && p <= MCE_MAX_P, p, x);
  }
  const u64 wiso = wave_sum_u64(iso);
  const u64 whash = wave_sum_u64(iso_hash);
  const u32 wpm = wave_max_u32((u32)pmax);
  const u32 wxm = wave_max_u32((u32)xmax);
  const u32 wl = wave_or_u32(lim);
  if (lane == 0) {
    if (wiso) {
      atomicAdd(&ctl->isolated, wiso);
      atomicAdd(&ctl->isolated_hash, whash);
    }
    atomicMax(&ctl->max_p, (int)wpm);
    atomicMax(&ctl->max_x, (int)wxm);
    if (wl & 1u) atomicOr(&ctl->status, MCE_E_LIMIT);
  }
  tally_end(s_tally, ctl);
}

// Scatter the roots with 1 <= |P| <= MCE_MAX_P into one list per sub-class of
// the chosen mode, starting at off[sub]. Each block takes a contiguous range of
// roots in two passes: it counts them per sub-class (LDS atomics, one per wave
// and sub-class), reserves its places with one device atomic per sub-class,
// then places them from LDS cursors. (One device atomic per wave and sub-class
// on the shared cursors cost a 500k-root run about 0.13 ms.)
__global__ __launch_bounds__(256) void k_bucket(const int* __restrict__ roots, int nroots,
                                                 const int* __restrict__ pcount, const int* __restrict__ xcount,
                                                 int mode, int micro, SubOffsets off, int* lists, u64* words,
                                                 MceCtl* ctl) {
  __shared__ int s_cnt[MCE_NSUB];
  __shared__ int s_cur[MCE_NSUB];
  __shared__ int s_ok;
  if (threadIdx.x == 0) s_ok = ld_relaxed(&ctl->status) == 0 ? 1 : 0;
  for (int i = threadIdx.x; i < MCE_NSUB; i += blockDim.x) s_cnt[i] = 0;
  __syncthreads();
  if (!s_ok) return;
  const int lane = lane_id();
  const int per = (nroots + gridDim.x - 1) / gridDim.x;
  const int r0 = min(nroots, blockIdx.x * per), r1 = min(nroots, r0 + per);
  for (int pass = 0; pass < 2; pass++) {
    for (int base = r0; base < r1; base += blockDim.x) {
      const int i = base + threadIdx.x;
      const int p = i < r1 ? pcount[i] : 0;
      const int x = i < r1 ? xcount[i] : 0;
      const bool valid = p > 0 && p <= MCE_MAX_P;
      const int sub = valid ? mce_sub_of(p, x, mode, micro != 0) : -1;
      u64 pending = ballot(valid);
      while (pending) {
        const int sc = read_lane(sub, __builtin_ctzll(pending));
        const bool mine = sub == sc;
        const u64 m = ballot(mine);
        pending &= ~m;
        if (pass == 0) {
          if (lane == 0) atomicAdd(&s_cnt[sc], __popcll(m));
        } else {
          int pos = 0;
          if (lane == 0) pos = atomicAdd(&s_cur[sc], __popcll(m));
          pos = read_lane(pos, 0);
          if (mine) {
            lists[off.off[sc] + pos + mbcnt(m)] = roots ? roots[i] : i;
            words[off.off[sc] + pos + mbcnt(m)] = mce_sub_table_words(p, x, sc, mode);
          }
        }
      }
    }
    if (pass == 0) {
      __syncthreads();
      for (int c = threadIdx.x; c < MCE_NSUB; c += blockDim.x)
        s_cur[c] = s_cnt[c] ? atomicAdd(&ctl->sub_cursor[c], s_cnt[c]) : 0;
      __syncthreads();
    }
  }
}

// Clears `words` u64 (the control block before a run). A kernel rather than a
// memset: the same stream operation, and one that a captured graph replays
// correctly.
__global__ __launch_bounds__(256) void k_zero(u64* p, long long words) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < words; i += (long long)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

// ------------------------------------------------------------------ launchers

hipError_t mce_launch_zero(u64* p, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  const int nb = (int)std::min<size_t>(64, (words + 255) / 256);
  hipLaunchKernelGGL(k_zero, dim3(nb), dim3(256), 0, s, p, (long long)words);
  return hipGetLastError();
}

hipError_t mce_launch_validate(int n, long long nnz, const int* rp, const int* ci, MceCtl* ctl, int blocks,
                               hipStream_t s) {
  if (n <= VAL_SMALL_N && nnz <= VAL_SMALL_NNZ) {
    hipLaunchKernelGGL(k_validate_small, dim3(1), dim3(1024), 0, s, n, nnz, rp, ci, ctl);
    return hipGetLastError();
  }
  int nb = max(1, min(blocks, (n + 255) / 256));
  hipLaunchKernelGGL(k_validate_rowptr, dim3(nb), dim3(256), 0, s, n, nnz, rp, ctl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // equal whole tiles of entries per wave, four waves per block
  const long long tiles = (nnz + MCE_WAVE - 1) / MCE_WAVE;
  const int nbw = (int)std::max(1LL, std::min((long long)blocks, (tiles + 3) / 4));
  const long long nw = 4LL * nbw;
  const int per_wave = (int)((tiles + nw - 1) / nw * MCE_WAVE);
  hipLaunchKernelGGL(k_validate_cols, dim3(nbw), dim3(256), 0, s, n, nnz, per_wave, rp, ci, ctl);
  return hipGetLastError();
}

hipError_t mce_launch_peel(int n, const int* rp, const int* ci, int* deg, int* rnd, int* core, int* alive0,
                           int* alive1, int* front0, int* front1, int* bfront0, int* bfront1, MceCtl* ctl,
                           u64 budget, unsigned short* tcol, long long tcap, int* tcrow, int blocks, int split,
                           unsigned char* snap, hipEvent_t handed, hipStream_t s) {
  if (!tcol || !tcrow) tcap = 0;
  tcap = tcap < 0 ? 0 : (tcap > 0x7FFFFFFFll ? 0x7FFFFFFFll : tcap);   // row offsets are int
  if (blocks == 1 || tcap == 0 || !snap) split = 0;
  void* args[] = {&n,      (void*)&rp, (void*)&ci, &deg,    &rnd,  &core, &alive0, &alive1, &front0, &front1,
                  &bfront0, &bfront1,  &ctl,       &budget, &tcol, &tcap, &tcrow,  &split,  &snap};
  // one block needs no grid barrier, hence no cooperative launch
  if (blocks == 1) return hipLaunchKernel((const void*)k_peel, dim3(1), dim3(PEEL_THREADS), args, 0, s);
  hipError_t e = hipLaunchCooperativeKernel((const void*)k_peel, dim3(blocks), dim3(PEEL_THREADS), args, 0, s);
  if (e != hipSuccess || !split) return e;
  if (handed && (e = hipEventRecord(handed, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_peel_tail, dim3(1), dim3(PEEL_THREADS), 0, s, n, rp, ci, deg, rnd, core, alive0, alive1,
                     front0, front1, bfront0, bfront1, ctl, budget, tcol, tcap, tcrow);
  return hipGetLastError();
}

// The peel's grid barrier needs every block resident: one block per CU, well
// inside the occupancy limit.
int mce_peel_tail_rows() { return PEEL_TT + 1; }

int mce_peel_max_blocks(int num_cu) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_peel, PEEL_THREADS, 0) != hipSuccess ||
      per_cu < 1)
    return 1;
  return num_cu;
}

// ------------------------------------------------------------------ second-level subtrees
// Section 3.2, Algorithm 4: one subtree per edge {v_i, v_j}; v_j the later end,
// R = {v_i, v_j}, P = the common neighbours after v_j, X = those before it. The
// roots of a run are the forward edges (v_i, v_j), v_j after v_i, of its vertex
// roots (a vertex of degree 0 is a clique of its own, counted by k_orient).

// The COO source of every CSR entry (the page keeps CSR+COO for second-level
// subtrees): one wavefront per row.
__global__ __launch_bounds__(256) void k_coo_src(int n, const int* __restrict__ rp, int* src) {
  const int lane = lane_id();
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / MCE_WAVE;
  const int nwaves = gridDim.x * blockDim.x / MCE_WAVE;
  for (int v = wave; v < n; v += nwaves)
    for (int e = rp[v] + lane; e < rp[v + 1]; e += MCE_WAVE) src[e] = v;
}

// The forward edges of every vertex root, as CSR positions, at the root's
// offset (an exclusive prefix sum of the later-neighbour counts). One wavefront
// per root; the wave of the last root writes the total.
__global__ __launch_bounds__(256) void k_l2_expand(int n, const int* __restrict__ rp, const int* __restrict__ ci,
                                                    const int* __restrict__ rnd, const int* __restrict__ roots,
                                                    int nroots, const u64* __restrict__ off, int* eroots,
                                                    MceCtl* ctl) {
  if (ld_relaxed(&ctl->status) != 0) return;
  const int lane = lane_id();
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / MCE_WAVE;
  const int nwaves = gridDim.x * blockDim.x / MCE_WAVE;
  for (int i = wave; i < nroots; i += nwaves) {
    const int r = roots ? roots[i] : i;
    const int a = rp[r], b = rp[r + 1];
    const int rr = rnd[r];
    int pos = (int)off[i];
    for (int base = a; base < b; base += MCE_WAVE) {
      const int e = base + lane;
      const bool lat = e < b && order_after(rnd[ci[e]], ci[e], rr, r);
      const u64 m = ballot(lat);
      if (lat) eroots[pos + mbcnt(m)] = e;
      pos += __popcll(m);
    }
    if (i == nroots - 1 && lane == 0) ctl->l2_roots = pos;
  }
}

// Hub adjacency bitmaps (second-level orientation). On power-law graphs most
// forward edges point at high-degree vertices, and testing an entry of the
// short row for membership in a hub's row took a binary search of about a
// dozen dependent loads; with one n-bit bitmap per hub it is one load. Hubs are
// the vertices of degree >= HUB_MIN_DEG, the first maxhubs of them by an atomic
// counter (which ones only changes the speed).
#define HUB_MIN_DEG 256
__global__ __launch_bounds__(256) void k_hub_pick(int n, const int* __restrict__ rp, int* hub_id, int* hub_v,
                                                   int maxhubs, MceCtl* ctl) {
  if (ld_relaxed(&ctl->status) != 0) return;
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < n; v += gridDim.x * blockDim.x) {
    int id = -1;
    if (rp[v + 1] - rp[v] >= HUB_MIN_DEG) {
      const int k = atomicAdd(&ctl->nhubs, 1);
      if (k < maxhubs) {
        id = k;
        hub_v[k] = v;
      }
    }
    hub_id[v] = id;
  }
}

// One block per hub: clear its bitmap (words u64), then set the bit of every neighbour.
__global__ __launch_bounds__(256) void k_hub_fill(const int* __restrict__ rp, const int* __restrict__ ci,
                                                   const int* __restrict__ hub_v, int maxhubs, int words, u64* bm,
                                                   MceCtl* ctl) {
  if (ld_relaxed(&ctl->status) != 0) return;
  const int nh = min(ld_relaxed(&ctl->nhubs), maxhubs);
  for (int h = blockIdx.x; h < nh; h += gridDim.x) {
    u64* b = bm + (size_t)h * words;
    for (int w = threadIdx.x; w < words; w += blockDim.x) b[w] = 0ull;
    __syncthreads();
    const int v = hub_v[h];
    for (int k = rp[v] + (int)threadIdx.x; k < rp[v + 1]; k += blockDim.x) {
      const int u = ci[k];
      atomicOr(&b[u >> 6], 1ull << (u & 63));
    }
    __syncthreads();
  }
}

// Per second-level root: |P| and |X| by intersecting the two rows (each entry
// of the shorter one is searched in the longer one), then the same tallies as
// k_orient. A wavefront takes G consecutive roots, four at a time: lane group
// q (16 lanes) intersects root t0 + q's rows, and lane t keeps root t's counts,
// so that a tally covers up to 64 roots. (One root per wavefront left most
// lanes idle through the search chains: the shorter row has a few dozen entries
// on these graphs.) Roots with P and X empty are maximal cliques of size 2,
// counted here.
#define L2_GROUP 16   // lanes per root
__global__ __launch_bounds__(256) void k_orient_l2(const int* __restrict__ rp, const int* __restrict__ ci,
                                                    const int* __restrict__ rnd, const int* __restrict__ src,
                                                    const int* __restrict__ eroots, int* pcount, int* xcount,
                                                    const int* __restrict__ hub_id, const u64* __restrict__ bm,
                                                    int words, MceCtl* ctl) {
  __shared__ TallyAcc s_tally;
  __shared__ int s_ok;
  if (!tally_begin(s_tally, &s_ok, ctl)) return;
  constexpr int NQ = MCE_WAVE / L2_GROUP;   // roots in flight per wavefront
  const int lane = lane_id();
  const int q = lane / L2_GROUP, sl = lane % L2_GROUP;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / MCE_WAVE;
  const int nwaves = gridDim.x * blockDim.x / MCE_WAVE;
  const int total = ld_relaxed(&ctl->l2_roots);
  const int G = max(8, min(MCE_WAVE, (total + nwaves - 1) / nwaves));   // 8: few tallies on small graphs
  u64 pairs = 0, pairs_hash = 0;
  u32 lim = 0;
  for (int g0 = wave * G; g0 < total; g0 += nwaves * G) {
    int p = 0, x = 0;
    bool mine = false;
    for (int t0 = 0; t0 < G && g0 + t0 < total; t0 += NQ) {
      const int t = t0 + q;
      const bool live = t < G && g0 + t < total;
      int vi = 0, vj = 0;
      u32 cp = 0, cx = 0;
      if (live) {
        const int e = eroots[g0 + t];
        vi = src[e];
        vj = ci[e];
        const int ai = rp[vi], bi = rp[vi + 1], aj = rp[vj], bj = rp[vj + 1];
        const bool si = bi - ai <= bj - aj;   // scan the shorter row
        const int sa = si ? ai : aj, sb = si ? bi : bj, oa = si ? aj : ai, ob = si ? bj : bi;
        const int rj = rnd[vj];
        const int hid = hub_id ? hub_id[si ? vj : vi] : -1;   // the longer row's owner: a hub?
        const u64* hb = bm + (size_t)(hid < 0 ? 0 : hid) * words;
        for (int k = sa + sl; k < sb; k += L2_GROUP) {
          const int c = ci[k];
          if (hid >= 0 ? ((hb[c >> 6] >> (c & 63)) & 1ull) != 0ull : csr_range_has(ci, oa, ob, c)) {
            if (order_after(rnd[c], c, rj, vj)) cp++;
            else cx++;
          }
        }
      }
      // group sums (every lane active again), then lane t takes root t's from its group
#pragma unroll
      for (int off = L2_GROUP / 2; off >= 1; off >>= 1) {
        cp += (u32)__shfl_xor((int)cp, off);
        cx += (u32)__shfl_xor((int)cx, off);
      }
      const bool take = lane >= t0 && lane < t0 + NQ;   // lane t = t0 + q' takes group q'
      const int from = take ? (lane - t0) * L2_GROUP : lane;
      const u32 gp = (u32)__shfl((int)cp, from), gx = (u32)__shfl((int)cx, from);
      const int gvi = __shfl(vi, from), gvj = __shfl(vj, from);
      if (take && lane < G && g0 + lane < total) {
        p = (int)gp;
        x = (int)gx;
        mine = true;
        if (gp == 0 && gx == 0) {
          pairs++;
          pairs_hash += mce_clique_term(mce_vertex_term(gvi) + mce_vertex_term(gvj), 2);
        }
      }
    }
    if (mine) {
      pcount[g0 + lane] = p;
      xcount[g0 + lane] = x;
      if (p > MCE_MAX_P) lim |= 1u;
    }
    tally_roots(s_tally, mine && p > 0 && p <= MCE_MAX_P, p, x);
  }
  const u64 wp = wave_sum_u64(pairs), wh = wave_sum_u64(pairs_hash);
  const u32 wl = wave_or_u32(lim);
  if (lane == 0) {
    if (wp) {
      atomicAdd(&ctl->pairs, wp);
      atomicAdd(&ctl->pairs_hash, wh);
    }
    if (wl) atomicOr(&ctl->status, MCE_E_LIMIT);
  }
  tally_end(s_tally, ctl);
}

hipError_t mce_launch_hubs(int n, const int* rp, const int* ci, int* hub_id, int* hub_v, u64* bm, int maxhubs,
                           MceCtl* ctl, int blocks, hipStream_t s) {
  const int words = (n + 63) / 64;
  const int nbh = (int)std::max(1LL, std::min((long long)blocks, ((long long)n + 255) / 256));
  hipLaunchKernelGGL(k_hub_pick, dim3(nbh), dim3(256), 0, s, n, rp, hub_id, hub_v, maxhubs, ctl);
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_hub_fill, dim3(std::max(1, std::min(blocks, maxhubs))), dim3(256), 0, s, rp, ci,
                     (const int*)hub_v, maxhubs, words, bm, ctl);
  return hipGetLastError();
}

hipError_t mce_launch_l2_roots(int n, long long nnz, const int* rp, const int* ci, const int* rnd,
                               const int* roots, int nroots, u64* fwd, u64* fwd_tmp, int* src, int* eroots,
                               int* pcount, int* xcount, int* hub_id, int* hub_v, u64* bm, int maxhubs,
                               MceCtl* ctl, int blocks, hipStream_t s) {
  hipError_t e;
  const int words = (n + 63) / 64;
  const int nbr = (int)std::max(1LL, std::min((long long)blocks, ((long long)n + 3) / 4));
  hipLaunchKernelGGL(k_coo_src, dim3(nbr), dim3(256), 0, s, n, rp, src);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mce_launch_scan(fwd, nroots, fwd_tmp, s)) != hipSuccess) return e;
  const int nbe = (int)std::max(1LL, std::min((long long)blocks, ((long long)nroots + 3) / 4));
  hipLaunchKernelGGL(k_l2_expand, dim3(nbe), dim3(256), 0, s, n, rp, ci, rnd, roots, nroots, (const u64*)fwd,
                     eroots, ctl);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nbo = (int)std::max(1LL, std::min((long long)blocks, nnz / 8 + 1));
  hipLaunchKernelGGL(k_orient_l2, dim3(nbo), dim3(256), 0, s, rp, ci, rnd, (const int*)src, (const int*)eroots,
                     pcount, xcount, maxhubs > 0 ? (const int*)hub_id : nullptr, (const u64*)bm, words, ctl);
  return hipGetLastError();
}

hipError_t mce_launch_search_rank(int n, const int* rnd, const int* deg, const unsigned char* snap,
                                  const MceCtl* tctl, int* srank, int blocks, hipStream_t s) {
  const int nb = max(1, min(blocks, (n + 255) / 256));
  hipLaunchKernelGGL(k_search_rank, dim3(nb), dim3(256), 0, s, n, rnd, deg, snap, tctl, srank);
  return hipGetLastError();
}

hipError_t mce_launch_orient_handover(int n, const int* rp, const int* fdeg, const MceCtl* tctl, int* pcount,
                                      int* xcount, MceCtl* ctl, int blocks, hipStream_t s) {
  const int nb = max(1, min(max(1, blocks / 8), (n + 255) / 256));
  hipLaunchKernelGGL(k_orient_handover, dim3(nb), dim3(256), 0, s, n, rp, fdeg, tctl, pcount, xcount, ctl);
  return hipGetLastError();
}

hipError_t mce_launch_orient(int n, const int* rp, const int* ci, const int* rnd, const int* roots, int nroots,
                             int* pcount, int* xcount, MceCtl* ctl, u64* fwd, const int* fdeg, int blocks,
                             hipStream_t s) {
  if (fdeg && (roots || fwd || nroots != n)) return hipErrorInvalidValue;   // every vertex a root, first level
  // at most one root per wavefront of the grid: a wavefront per root, on at most
  // 256 wavefronts (every wavefront ends with a few atomics on the same words:
  // thousands of them cost more than walking several rows each)
  const int per_wave = !fdeg && nroots <= 4 * blocks ? 1 : 0;
  // (a thread per root otherwise; each block adds its tallies to the control
  // block once, so with |P| read from fdeg, where a thread does little else,
  // fewer blocks take more roots each)
  const int tb = fdeg ? max(1, blocks / 8) : blocks;
  const int nb = per_wave ? max(1, min(64, (nroots + 3) / 4)) : max(1, min(tb, (nroots + 255) / 256));
  hipLaunchKernelGGL(k_orient, dim3(nb), dim3(256), 0, s, n, rp, ci, rnd, roots, nroots, pcount, xcount, ctl, fwd,
                     fdeg, fwd ? 0 : 1, per_wave, ORIENT_MUL);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !per_wave || fwd) return e;
  hipLaunchKernelGGL(k_tally, dim3(max(1, min(blocks, (nroots + 255) / 256))), dim3(256), 0, s, nroots, pcount,
                     xcount, ctl);
  return hipGetLastError();
}

hipError_t mce_launch_forward_adj(int n, const int* rp, const int* ci, const int* rnd, int* fadj, int* fdeg,
                                  int* flong, MceCtl* ctl, int blocks, hipStream_t s, const MceCtl* tctl) {
  const int nb = max(1, min(blocks, (n + 3) / 4));   // four wavefronts a block, one vertex each at a time
  hipLaunchKernelGGL(k_forward_adj, dim3(nb), dim3(256), 0, s, n, rp, ci, rnd, fadj, fdeg, flong, ctl, tctl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_forward_adj_long, dim3(max(1, blocks)), dim3(256), 0, s, rp, ci, rnd, fadj, fdeg, flong, ctl,
                     tctl);
  return hipGetLastError();
}

hipError_t mce_launch_bucket(const int* roots, int nroots, const int* pcount, const int* xcount, int mode,
                             int micro, SubOffsets off, int* lists, u64* words, MceCtl* ctl, int blocks,
                             hipStream_t s) {
  // (at most blocks / 8 blocks, each over a contiguous range of roots)
  const int nb = max(1, min(max(1, blocks / 8), (nroots + 255) / 256));
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
