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
// memory operations completed, then arrives, and the last arrival opens the next
// generation. Bounded: past the deadline it flags MCE_E_TIMEOUT and lets the
// block go; the caller checks the flag after every barrier.
__device__ void grid_sync(MceCtl* ctl, u64 deadline) {
  wait_stores_complete();
  __syncthreads();
  if (gridDim.x > 1) {
    if (threadIdx.x == 0) {
      const u32 gen = ld_relaxed(&ctl->bar_gen);
      wait_stores_complete();   // the generation is read before this block arrives
      const u32 arrived = __hip_atomic_fetch_add(&ctl->bar_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
      if (arrived == gridDim.x) {
        st_relaxed(&ctl->bar_count, 0u);
        wait_stores_complete();
        st_relaxed(&ctl->bar_gen, gen + 1);
      } else {
        u32 spins = 0;
        while (ld_relaxed(&ctl->bar_gen) == gen) {
          __builtin_amdgcn_s_sleep(1);
          if ((++spins & 1023u) == 0 && past_deadline(deadline)) {
            atomicOr(&ctl->status, MCE_E_TIMEOUT);
            break;
          }
        }
      }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ int ldi(const int* p) { return ld_relaxed(p); }
__device__ __forceinline__ void sti(int* p, int v) { st_relaxed_i(p, v); }

// Round-synchronous peel (section 2.4 asks for a degeneracy order; this is the
// one the engine uses). Level k: every remaining vertex of current degree <= k
// leaves in one round (rnd = round, core = k). The removed vertices' remaining
// neighbours lose one degree each, and a neighbour whose degree falls from k+1
// to k joins the next round of the same level; when a round removes nothing, k
// becomes the smallest remaining degree. Marking the round's vertices and
// decrementing their neighbours happen in the same phase: a vertex of the
// current round already has degree <= k, so a decrement can never make it join
// again (that needs a fall from k+1). One grid barrier per round. Launched
// cooperatively; one block for small graphs.
__global__ __launch_bounds__(256) void k_peel(int n, const int* __restrict__ rp, const int* __restrict__ ci,
                                               int* deg, int* rnd, int* core, int* alive0, int* alive1,
                                               int* front0, int* front1, MceCtl* ctl, u64 budget) {
  if (ld_relaxed(&ctl->status) != 0) return;   // rejected input: nothing to order
  const u64 t0 = wall_clock64();
  const u64 deadline = t0 + budget;
  const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
  const int gsize = gridDim.x * blockDim.x;
  const int lane = lane_id();
  const int wave = gtid / MCE_WAVE;
  const int nwaves = gsize / MCE_WAVE;
  int* alive[2] = {alive0, alive1};
  int* front[2] = {front0, front1};

  for (int v = gtid; v < n; v += gsize) {
    sti(&deg[v], rp[v + 1] - rp[v]);
    sti(&rnd[v], -1);
    sti(&alive0[v], v);
  }
  if (gtid == 0) {
    st_relaxed64(&ctl->t_run, t0);
    sti(&ctl->asize[0], n);
    sti(&ctl->asize[1], 0);
    sti(&ctl->fsize[0], 0);
    sti(&ctl->fsize[1], 0);
    sti(&ctl->fsize[2], 0);
    sti(&ctl->min_deg, 0x7FFFFFFF);
  }
  grid_sync(ctl, deadline);

  int cur = 0, nf = 0, k = 0, r = 0;
  int na = n;
  for (;;) {
    if (ld_relaxed(&ctl->status) & MCE_E_TIMEOUT) return;
    if (nf == 0) {
      // new level: compact the remaining list and find the smallest remaining degree
      const int* src = alive[cur];
      int* dst = alive[cur ^ 1];
      int mn = 0x7FFFFFFF;
      for (int base = wave * MCE_WAVE; base < na; base += nwaves * MCE_WAVE) {
        const int i = base + lane;
        bool keep = false;
        int v = 0;
        if (i < na) {
          v = ldi(&src[i]);
          keep = ldi(&rnd[v]) < 0;
          if (keep) mn = min(mn, ldi(&deg[v]));
        }
        const u64 m = ballot(keep);
        int pos = 0;
        if (lane == 0 && m) pos = atomicAdd(&ctl->asize[cur ^ 1], __popcll(m));
        pos = read_lane(pos, 0);
        if (keep) sti(&dst[pos + mbcnt(m)], v);
      }
      const int wmn = wave_min_i32_nonneg(mn);
      if (lane == 0 && wmn != 0x7FFFFFFF) atomicMin(&ctl->min_deg, wmn);
      grid_sync(ctl, deadline);
      if (ld_relaxed(&ctl->status) & MCE_E_TIMEOUT) return;
      cur ^= 1;
      na = ldi(&ctl->asize[cur]);
      if (na == 0) break;
      k = ldi(&ctl->min_deg);
      // the level's first round: every remaining vertex of degree <= k
      const int* al = alive[cur];
      int* fr = front[r & 1];
      for (int base = wave * MCE_WAVE; base < na; base += nwaves * MCE_WAVE) {
        const int i = base + lane;
        bool in = false;
        int v = 0;
        if (i < na) {
          v = ldi(&al[i]);
          in = ldi(&deg[v]) <= k;
        }
        const u64 m = ballot(in);
        int pos = 0;
        if (lane == 0 && m) pos = atomicAdd(&ctl->fsize[r % 3], __popcll(m));
        pos = read_lane(pos, 0);
        if (in) sti(&fr[pos + mbcnt(m)], v);
      }
      grid_sync(ctl, deadline);
      if (ld_relaxed(&ctl->status) & MCE_E_TIMEOUT) return;
      nf = ldi(&ctl->fsize[r % 3]);
    }
    // round r: remove the frontier, take one degree from each remaining neighbour
    if (gtid == 0) {
      // counters nobody reads any more: the frontier size read two rounds ago,
      // the old remaining-list size and the level's minimum
      sti(&ctl->fsize[(r + 2) % 3], 0);
      sti(&ctl->asize[cur ^ 1], 0);
      sti(&ctl->min_deg, 0x7FFFFFFF);
    }
    const int* fr = front[r & 1];
    int* nx = front[(r + 1) & 1];
    int* nxs = &ctl->fsize[(r + 1) % 3];
    for (int i = wave; i < nf; i += nwaves) {
      const int v = ldi(&fr[i]);
      if (lane == 0) {
        sti(&rnd[v], r);
        core[v] = k;
      }
      const int a = rp[v], b = rp[v + 1];
      for (int base = a; base < b; base += MCE_WAVE) {
        const int e = base + lane;
        bool joins = false;
        int u = 0;
        if (e < b) {
          u = ci[e];
          if (ldi(&rnd[u]) < 0) joins = atomicSub(&deg[u], 1) == k + 1;
        }
        const u64 m = ballot(joins);
        int pos = 0;
        if (lane == 0 && m) pos = atomicAdd(nxs, __popcll(m));
        pos = read_lane(pos, 0);
        if (joins) sti(&nx[pos + mbcnt(m)], u);
      }
    }
    grid_sync(ctl, deadline);
    if (ld_relaxed(&ctl->status) & MCE_E_TIMEOUT) return;
    nf = ldi(nxs);
    r++;
  }
  if (gtid == 0) {
    ctl->rounds = r;
    ctl->degeneracy = k;
  }
}

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
                                                 int mode, int micro, SubOffsets off, int* lists, MceCtl* ctl) {
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
      if (mine) lists[off.off[s] + pos + mbcnt(m)] = roots ? roots[i] : i;
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
                           int* alive1, int* front0, int* front1, MceCtl* ctl, u64 budget, int blocks,
                           hipStream_t s) {
  void* args[] = {&n, (void*)&rp, (void*)&ci, &deg, &rnd, &core, &alive0, &alive1,
                  &front0, &front1, &ctl, &budget};
  return hipLaunchCooperativeKernel((const void*)k_peel, dim3(blocks), dim3(256), args, 0, s);
}

// The peel's grid barrier needs every block resident: stay well inside the
// occupancy limit (two 256-thread blocks per CU keep the streaming passes at
// full bandwidth).
int mce_peel_max_blocks(int num_cu) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_peel, 256, 0) != hipSuccess)
    return 1;
  return max(1, min(per_cu, 2) * num_cu);
}

hipError_t mce_launch_orient(int n, const int* rp, const int* ci, const int* rnd, const int* roots, int nroots,
                             int* pcount, int* xcount, MceCtl* ctl, int blocks, hipStream_t s) {
  const int nb = max(1, min(blocks, (nroots + 255) / 256));
  hipLaunchKernelGGL(k_orient, dim3(nb), dim3(256), 0, s, n, rp, ci, rnd, roots, nroots, pcount, xcount, ctl);
  return hipGetLastError();
}

hipError_t mce_launch_bucket(const int* roots, int nroots, const int* pcount, const int* xcount, int mode,
                             int micro, SubOffsets off, int* lists, MceCtl* ctl, int blocks, hipStream_t s) {
  const int nb = max(1, min(blocks, (nroots + 255) / 256));
  hipLaunchKernelGGL(k_bucket, dim3(nb), dim3(256), 0, s, roots, nroots, pcount, xcount, mode, micro, off, lists,
                     ctl);
  return hipGetLastError();
}
