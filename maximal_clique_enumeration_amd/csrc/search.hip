// The search: Bron-Kerbosch with pivoting over independent first-level subtrees,
// one wavefront per subtree, as a single persistent launch per bitset-width
// class.
//
// "Parallelizing Maximal Clique Enumeration on GPUs" (arxiv 2212.01473v2):
//  - section 2.3, Algorithm 2: branch on P - N(pivot); after a branch on v,
//    P = P - {v} and X = X u {v}; R is maximal when P and X are both empty;
//  - section 2.4, Algorithm 3: subtree of v_i starts from ({v_i}, later
//    neighbours, earlier neighbours) under a degeneracy order;
//  - section 3.1: a block walks its subtree depth-first, its threads sharing the
//    set operations and the pivot search; section 3.3: persistent blocks take
//    subtrees from a shared counter, then idle blocks wait in a worker list and
//    busy blocks donate branches (only if |P| >= threshold and unexplored
//    branches remain at this level and at a shallower one);
//  - section 3.4: partial induced subgraph -- bit-encoded rows for P x P only,
//    P-X edges looked up in the CSR; section 3.5: X split into X_P (bitset, one
//    copy per level) and X_X (one array for all levels, shrinking, with an end
//    index lpX per level); the pivot then comes from X_P u P only.
//
// MI355X mapping: the "block" is one 64-lane wavefront. A P bitset of W 64-bit
// words lives in lanes 0..W-1; the pivot evaluates one candidate row per lane
// (AND + popcount over W words) and takes a DPP max-reduction of a packed
// (count, index) key; child sets are W-lane ANDs; the X_X filter is a
// ballot/mbcnt stable partition over 64 entries at a time.
#include "mce_device.h"
#include "mce_internal.h"

#define REC_WORDS(W) (3 * (W) + 2)   // per level: P[W], X_P[W], C[W], s, (lpX | open << 32)

template <int W>
struct Dims {
  static constexpr int PMAX = 64 * W;            // largest |P_root| of the class
  static constexpr int HCAP = PMAX + 2;          // clique sizes 0..PMAX+1
  static constexpr int REC = REC_WORDS(W);
  static constexpr int LEVELS = PMAX + 1;        // |P| drops by >= 1 per level
  static constexpr int MAIL = 3 + 2 * W;         // mailbox words
};

// ------------------------------------------------------------------ worker list
// Receiver side (section 3.3): give up this wave's share of n_active. The wave
// that brings it to zero after the roots ran out ends the launch (no task is
// held anywhere and none can appear, since only active waves donate). Any other
// wave publishes its id and spins on its wake flag with exponential back-off.
// Returns 1 with a task in the mailbox (the donor re-counted this wave as
// active), 0 to exit.
__device__ int wl_wait(MceWl* wl, int wid, u64 deadline, u32* status) {
  int res = 0;
  if (lane_id() == 0) {
    int left = __hip_atomic_fetch_add(&wl->n_active, -1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) - 1;
    if (left <= 0) {
      if (left < 0) atomicOr(status, MCE_E_PROTO);
      st_release(&wl->done, 1u);
    } else {
      st_relaxed(&wl->flag[wid], 0u);
      __hip_atomic_fetch_or(&wl->idle_bits[wid >> 6], 1ull << (wid & 63), __ATOMIC_RELEASE,
                            __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&wl->n_waiting, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int backoff = 1;
      u32 it = 0;
      for (;;) {
        if (ld_relaxed(&wl->flag[wid])) {
          res = 1;
          break;
        }
        if (ld_relaxed(&wl->done)) break;
        if ((++it & 7u) == 0 && past_deadline(deadline)) {
          atomicOr(status, MCE_E_TIMEOUT);
          st_release(&wl->done, 1u);
          break;
        }
        for (int i = 0; i < backoff; i++) __builtin_amdgcn_s_sleep(4);
        if (backoff < 16) backoff <<= 1;
      }
    }
  }
  res = read_lane(res, 0);
  fence_acquire_agent();
  return res;
}

// Donor side: take one idle wavefront out of the bitmap, or -1. The claimed
// wave is counted active before the donor can ever give up its own share, so
// n_active cannot reach zero while the donated branch is in flight.
__device__ int wl_claim(MceWl* wl, int wid, int nworkers) {
  int r = -1;
  if (lane_id() == 0) {
    if (ld_relaxed(&wl->n_waiting) > 0) {
      int nw = (nworkers + 63) >> 6;
      int start = wid >> 6;
      for (int t = 0; t < nw && r < 0; t++) {
        int j = start + t;
        if (j >= nw) j -= nw;
        u64 word = ld_relaxed(&wl->idle_bits[j]);
        while (word) {
          int b = __builtin_ctzll(word);
          u64 bit = 1ull << b;
          u64 old = __hip_atomic_fetch_and(&wl->idle_bits[j], ~bit, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
          if (old & bit) {
            r = j * 64 + b;
            break;
          }
          word = old & ~bit;
        }
      }
      if (r >= 0) {
        __hip_atomic_fetch_add(&wl->n_waiting, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(&wl->n_active, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  return read_lane(r, 0);
}

// ------------------------------------------------------------------ X_X partition
// Stable in-place partition of xx[0, L): entries adjacent to vertex vg move to the
// front in their order, the others after them (section 3.5, Figure 2). Returns
// the number kept. Each 64-entry chunk is read whole before any of it is written:
// kept entries go to [wk, wk+kc); removed entries that sat there move, with the
// chunk's removed entries, to the tail of [wk, c+64).
__device__ int xx_partition(int* xx, int L, int vg, const int* __restrict__ rp, const int* __restrict__ ci,
                            u64& tests) {
  const int lane = lane_id();
  const int va = rp[vg], vb = rp[vg + 1];
  const int vdeg = vb - va;
  int wk = 0;
  for (int c = 0; c < L; c += MCE_WAVE) {
    int i = c + lane;
    bool valid = i < L;
    int x = valid ? xx[i] : 0;
    int kc_bound = min(MCE_WAVE, c - wk);
    int dval = lane < kc_bound ? xx[wk + lane] : 0;
    bool keep = false;
    if (valid) {
      int xa = rp[x], xb = rp[x + 1];
      keep = (xb - xa <= vdeg) ? csr_range_has(ci, xa, xb, vg) : csr_range_has(ci, va, vb, x);
    }
    u64 km = ballot(keep);
    u64 vm = ballot(valid);
    int kc = __popcll(km);
    int D = min(kc, c - wk);
    int base = max(c, wk + kc);
    __syncthreads();   // every lane has its values before anything is written
    if (keep) xx[wk + mbcnt(km)] = x;
    if (lane < D) xx[base + lane] = dval;
    if (valid && !keep) xx[base + D + mbcnt(vm & ~km)] = x;
    wk += kc;
    __syncthreads();
  }
  tests += (u64)L;
  return wk;
}

// Is any entry of xx[0, L) adjacent to vg? (X_X n N(v) empty test for a leaf.)
__device__ bool xx_any_adjacent(const int* xx, int L, int vg, const int* __restrict__ rp,
                                const int* __restrict__ ci, u64& tests) {
  const int lane = lane_id();
  const int va = rp[vg], vb = rp[vg + 1];
  const int vdeg = vb - va;
  for (int c = 0; c < L; c += MCE_WAVE) {
    int i = c + lane;
    bool hit = false;
    if (i < L) {
      int x = xx[i];
      int xa = rp[x], xb = rp[x + 1];
      hit = (xb - xa <= vdeg) ? csr_range_has(ci, xa, xb, vg) : csr_range_has(ci, va, vb, x);
    }
    tests += (u64)min(MCE_WAVE, L - c);
    if (ballot(hit)) return true;
  }
  return false;
}

// ------------------------------------------------------------------ the kernel
template <int W, bool LROWS, bool LSTACK>
__global__ __launch_bounds__(64) void k_search(SearchParams prm) {
  using D = Dims<W>;
  constexpr int PMAX = D::PMAX;
  constexpr int HCAP = D::HCAP;
  constexpr int REC = D::REC;
  extern __shared__ u64 lds[];

  const int lane = lane_id();
  const int wid = blockIdx.x;
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ ci = prm.ci;
  const int* __restrict__ rnd = prm.rnd;
  MceWl* wl = prm.wl;
  const u64 deadline = wall_clock64() + prm.budget;

  char* slot = prm.slots + (size_t)wid * prm.slot_bytes;
  int* xx = (int*)(slot + prm.off_xx);
  u64* mail = (u64*)(slot + prm.off_mail);

  u64* s_hist = lds;
  u64* rows;
  u64* hv;
  int* pid;
  u64* stk;
  if constexpr (LROWS) {
    rows = lds + HCAP;
    hv = rows + PMAX * W;
    pid = (int*)(hv + PMAX);
  } else {
    rows = (u64*)(slot + prm.off_rows);
    hv = (u64*)(slot + prm.off_hv);
    pid = (int*)(slot + prm.off_pid);
  }
  if constexpr (LSTACK) {
    stk = lds + HCAP + (LROWS ? (PMAX * W + PMAX + PMAX / 2) : 0);
  } else {
    stk = (u64*)(slot + prm.off_stack);
  }

  for (int i = lane; i < HCAP; i += MCE_WAVE) s_hist[i] = 0;
  __syncthreads();

  u64 hacc = 0;
  u64 st_nodes = 0, st_leaves = 0, st_don = 0, st_prow = 0, st_xx = 0, st_ip = 0, st_roots = 0, st_recv = 0;
  u64 idle_ticks = 0;
  const u64 t_start = wall_clock64();
  bool phase2 = false;
  bool abort = false;
  // this wave is active until phase 1 finds the roots exhausted (wl_wait gives
  // the share back)
  if (lane == 0) __hip_atomic_fetch_add(&wl->n_active, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  for (;;) {
    // ---------------------------------------------------------- get a task
    int p = 0, k0 = 0;
    if (!phase2) {
      u32 idx = 0;
      if (lane == 0) idx = atomicAdd(&wl->root_ctr, 1u);
      idx = (u32)read_lane((int)idx, 0);
      if (idx >= (u32)prm.nroots) {
        phase2 = true;
        continue;
      }
      // Build the root's task: split N(r) into P_root (later, ascending id) and
      // X_X (earlier), then the P x P bit rows (section 3.4).
      const int r = prm.roots[idx];
      const int a = rp[r], b = rp[r + 1];
      const int rr = rnd[r];
      int np = 0, nx = 0;
      for (int base = a; base < b; base += MCE_WAVE) {
        int e = base + lane;
        bool valid = e < b;
        int u = valid ? ci[e] : 0;
        bool lat = valid && order_after(rnd[u], u, rr, r);
        u64 lm = ballot(lat);
        u64 xm = ballot(valid && !lat);
        if (lat) {
          int pos = np + mbcnt(lm);
          if (pos < PMAX) pid[pos] = u;
        }
        if (valid && !lat) xx[nx + mbcnt(xm)] = u;
        np += __popcll(lm);
        nx += __popcll(xm);
      }
      if (np > PMAX || np == 0) {   // the host only sends 1 <= |P| <= PMAX here
        if (lane == 0) atomicOr(prm.status, MCE_E_LIMIT);
        continue;
      }
      p = np;
      k0 = 1;
      __syncthreads();
      for (int i = lane; i < p; i += MCE_WAVE) hv[i] = mce_vertex_term(pid[i]);
      for (int i = 0; i < p; i++) {
        const int gi = pid[i];
        const int ra = rp[gi], rb = rp[gi + 1];
#pragma unroll
        for (int w = 0; w < W; w++) {
          int j = w * 64 + lane;
          bool bit = j < p && j != i && csr_range_has(ci, ra, rb, pid[j]);
          u64 word = ballot(bit);
          if (lane == 0) rows[i * W + w] = word;
        }
      }
      u64* R0 = stk;
      if (lane < W) {
        int lo = lane * 64;
        int cnt = p - lo;
        u64 m = cnt <= 0 ? 0ull : (cnt >= 64 ? ~0ull : ((1ull << cnt) - 1));
        R0[lane] = m;
        R0[W + lane] = 0;
      }
      if (lane == 0) {
        R0[3 * W] = mce_vertex_term(r);
        R0[3 * W + 1] = (u64)(u32)nx;
      }
      st_ip += (u64)p;
      st_roots++;
      __syncthreads();
    } else {
      if (!prm.worker_list) break;
      u64 t0 = wall_clock64();
      int got = wl_wait(wl, wid, deadline, prm.status);
      idle_ticks += wall_clock64() - t0;
      if (!got) break;
      // a donor filled the mailbox and this slot's rows, hv, pid and xx
      u64 h0 = mail[0];
      p = (int)(u32)h0;
      k0 = (int)(h0 >> 32);
      int lpx = (int)(u32)mail[1];
      u64 s0 = mail[2];
      if constexpr (LROWS) {
        const u64* g_rows = (const u64*)(slot + prm.off_rows);
        const u64* g_hv = (const u64*)(slot + prm.off_hv);
        const int* g_pid = (const int*)(slot + prm.off_pid);
        for (int i = lane; i < p * W; i += MCE_WAVE) rows[i] = g_rows[i];
        for (int i = lane; i < p; i += MCE_WAVE) {
          hv[i] = g_hv[i];
          pid[i] = g_pid[i];
        }
      }
      u64* R0 = stk;
      if (lane < W) {
        R0[lane] = mail[3 + lane];
        R0[W + lane] = mail[3 + W + lane];
      }
      if (lane == 0) {
        R0[3 * W] = s0;
        R0[3 * W + 1] = (u64)(u32)lpx;
      }
      st_recv++;
      __syncthreads();
    }

    // ---------------------------------------------------------- depth-first search
    u64 myrow = 0;   // W == 1: candidate row `lane` kept in a register
    if constexpr (W == 1) {
      if (lane < p) myrow = rows[lane];
    }
    int l = 0;
    bool need_pivot = true;
    for (;;) {
      u64* R = stk + (size_t)l * REC;
      if (need_pivot) {
        need_pivot = false;
        st_nodes++;
        if ((st_nodes & 1023u) == 0) {
          int stop = 0;
          if (lane == 0) {
            if (ld_relaxed(&wl->done)) stop = 1;
            else if (past_deadline(deadline)) {
              atomicOr(prm.status, MCE_E_TIMEOUT);
              st_release(&wl->done, 1u);
              stop = 1;
            }
          }
          if (read_lane(stop, 0)) {
            abort = true;
            break;
          }
        }
        // Tomita pivot from P u X_P (section 3.5, last paragraph): the row with
        // the most P neighbours; ties to the smallest index (= smallest id).
        u64 pj = 0, xj = 0;
        if (lane < W) {
          pj = R[lane];
          xj = R[W + lane];
        }
        u32 best = 0;
#pragma unroll
        for (int wb = 0; wb < W; wb++) {
          const u64 cw = read_lane(pj | xj, wb);
          if (cw == 0) continue;
          st_prow += (u64)__popcll(cw);
          const int i = wb * 64 + lane;
          if ((cw >> lane) & 1ull) {
            u32 c = 0;
            if constexpr (W == 1) {
              c = (u32)__popcll(read_lane(pj, 0) & myrow);
            } else {
              const u64* row = rows + (size_t)i * W;
#pragma unroll
              for (int w = 0; w < W; w++) c += (u32)__popcll(read_lane(pj, w) & row[w]);
            }
            u32 key = (c << 11) | (u32)(2047 - i);
            best = best > key ? best : key;
          }
        }
        best = wave_max_u32(best);
        const int u = 2047 - (int)(best & 2047u);
        u64 cj = 0;
        if constexpr (W == 1) {
          if (lane == 0) cj = pj & ~read_lane(myrow, u);
          cj = read_lane(cj, 0);
          if (lane == 0) R[2] = cj;
        } else {
          if (lane < W) {
            cj = pj & ~rows[(size_t)u * W + lane];
            R[2 * W + lane] = cj;
          }
        }
        __syncthreads();
      }

      // next branch of this level: lowest vertex of C = P - N(pivot)
      u64 cj = 0, pj = 0, xj = 0;
      if (lane < W) {
        cj = R[2 * W + lane];
        pj = R[lane];
        xj = R[W + lane];
      }
      const u64 nz = ballot(lane < W && cj != 0);
      if (nz == 0) {
        if (l == 0) break;
        l--;
        continue;
      }
      const int j0 = __builtin_ctzll(nz);
      const u64 cw = read_lane(cj, j0);
      const int v = j0 * 64 + __builtin_ctzll(cw);
      const u64 vbit = cw & (~cw + 1);
      const bool more_here = (nz & ~(1ull << j0)) != 0 || (cw & (cw - 1)) != 0;
      u64 rv;
      if constexpr (W == 1) rv = read_lane(myrow, v);
      else rv = lane < W ? rows[(size_t)v * W + lane] : 0;
      const u64 pn = pj & rv;   // P n N(v)
      const u64 xn = xj & rv;   // X_P n N(v)
      if (lane == j0) {         // C -= {v}; P -= {v}; X_P += {v} (Algorithm 2)
        R[2 * W + j0] = cj & ~vbit;
        R[j0] = pj & ~vbit;
        R[W + j0] = xj | vbit;
      }
      const u64 meta = R[3 * W + 1];
      const int lpx = (int)(u32)meta;
      const int open = (int)(meta >> 32);
      const u64 s_child = R[3 * W] + hv[v];
      const int k_child = k0 + l + 1;
      const bool p_empty = ballot(lane < W && pn != 0) == 0;
      __syncthreads();
      if (p_empty) {
        const bool xp_empty = ballot(lane < W && xn != 0) == 0;
        if (xp_empty && !xx_any_adjacent(xx, lpx, pid[v], rp, ci, st_xx)) {
          // R u {v} is maximal: P and X are both empty
          hacc += mce_clique_term(s_child, k_child);
          if (lane == 0) s_hist[k_child] += 1;
          st_leaves++;
        }
        continue;
      }
      // X_X n N(v): stable partition, the child's part is xx[0, lpx_child)
      const int lpx_child = lpx > 0 ? xx_partition(xx, lpx, pid[v], rp, ci, st_xx) : 0;

      // donate this branch to an idle wavefront? (section 3.3 conditions)
      if (prm.worker_list && more_here && open > 0) {
        u32 pc = wave_sum_u32(lane < W ? (u32)__popcll(pn) : 0u);
        if ((int)pc >= prm.donate_min_p) {
          const int rcv = wl_claim(wl, wid, prm.nworkers);
          if (rcv >= 0) {
            char* dslot = prm.slots + (size_t)rcv * prm.slot_bytes;
            u64* d_rows = (u64*)(dslot + prm.off_rows);
            u64* d_hv = (u64*)(dslot + prm.off_hv);
            int* d_pid = (int*)(dslot + prm.off_pid);
            int* d_xx = (int*)(dslot + prm.off_xx);
            u64* d_mail = (u64*)(dslot + prm.off_mail);
            for (int i = lane; i < p * W; i += MCE_WAVE) d_rows[i] = rows[i];
            for (int i = lane; i < p; i += MCE_WAVE) {
              d_hv[i] = hv[i];
              d_pid[i] = pid[i];
            }
            for (int i = lane; i < lpx_child; i += MCE_WAVE) d_xx[i] = xx[i];
            if (lane < W) {
              d_mail[3 + lane] = pn;
              d_mail[3 + W + lane] = xn;
            }
            if (lane == 0) {
              d_mail[0] = (u64)(u32)p | ((u64)(u32)k_child << 32);
              d_mail[1] = (u64)(u32)lpx_child;
              d_mail[2] = s_child;
            }
            fence_release_agent();
            __syncthreads();
            if (lane == 0) st_release(&wl->flag[rcv], 1u);
            st_don++;
            continue;
          }
        }
      }
      // descend
      u64* Rn = R + REC;
      if (lane < W) {
        Rn[lane] = pn;
        Rn[W + lane] = xn;
      }
      if (lane == 0) {
        Rn[3 * W] = s_child;
        Rn[3 * W + 1] = (u64)(u32)lpx_child | ((u64)(u32)(open + (more_here ? 1 : 0)) << 32);
      }
      __syncthreads();
      l++;
      need_pivot = true;
    }
    if (abort) break;
  }

  // ---------------------------------------------------------- flush
  const u64 t_end = wall_clock64();
  if (!abort) {
    __syncthreads();
    for (int i = lane; i < HCAP; i += MCE_WAVE) {
      u64 h = s_hist[i];
      if (h) atomicAdd(&prm.g_hist[i], h);
    }
    if (lane == 0 && hacc) atomicAdd(prm.g_hash, hacc);
  }
  if (lane == 0) {
    u64* st = prm.stats + (size_t)wid * MCE_NSTAT;
    st[ST_NODES] = st_nodes;
    st[ST_LEAVES] = st_leaves;
    st[ST_DONATIONS] = st_don;
    st[ST_PIVOT_ROWS] = st_prow;
    st[ST_PIVOT_WORDS] = st_prow * (u64)W;
    st[ST_XX_TESTS] = st_xx;
    st[ST_IP_ROWS] = st_ip;
    st[ST_BUSY_TICKS] = (t_end - t_start) - idle_ticks;
    st[ST_ROOTS] = st_roots;
    st[ST_RECEIVED] = st_recv;
    st[ST_TOTAL_TICKS] = t_end - t_start;
  }
}

// Worker-list reset before a launch: every word zero.
__global__ void k_wl_init(MceWl* wl) {
  u32* w = (u32*)wl;
  const int nw = (int)(sizeof(MceWl) / 4);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nw; i += gridDim.x * blockDim.x) w[i] = 0;
}

// ------------------------------------------------------------------ host side
hipError_t mce_launch_wl_init(MceWl* wl, hipStream_t s) {
  hipLaunchKernelGGL(k_wl_init, dim3(1), dim3(1024), 0, s, wl);
  return hipGetLastError();
}

bool mce_search_lds_rows(int wclass) { return wclass <= 1; }    // W <= 2
bool mce_search_lds_stack(int wclass) { return wclass == 0; }   // W == 1

size_t mce_search_lds_bytes(int wclass, bool lds_rows, bool lds_stack) {
  const int W = 1 << wclass;
  const int PMAX = 64 * W;
  size_t words = (size_t)PMAX + 2;                                  // histogram
  if (lds_rows) words += (size_t)PMAX * W + PMAX + PMAX / 2;        // rows, hv, pid
  if (lds_stack) words += (size_t)(PMAX + 1) * REC_WORDS(W);
  return words * 8;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SlotLayout mce_slot_layout(int wclass, int max_x) {
  const int W = 1 << wclass;
  const int PMAX = 64 * W;
  SlotLayout L;
  size_t o = 0;
  L.off_rows = o;
  o = align256(o + (size_t)PMAX * W * 8);
  L.off_hv = o;
  o = align256(o + (size_t)PMAX * 8);
  L.off_pid = o;
  o = align256(o + (size_t)PMAX * 4);
  L.off_stack = o;
  o = align256(o + (size_t)(PMAX + 1) * REC_WORDS(W) * 8);
  L.off_mail = o;
  o = align256(o + (size_t)(3 + 2 * W) * 8);
  L.off_xx = o;
  o = align256(o + (size_t)(max_x > 0 ? max_x : 1) * 4);
  L.bytes = o;
  return L;
}

template <int W, bool LR, bool LS>
static const void* search_fn() {
  return (const void*)k_search<W, LR, LS>;
}

static const void* search_kernel(int wclass, bool hbm) {
  switch (wclass) {
    case 0: return hbm ? search_fn<1, false, false>() : search_fn<1, true, true>();
    case 1: return hbm ? search_fn<2, false, false>() : search_fn<2, true, false>();
    case 2: return search_fn<4, false, false>();
    case 3: return search_fn<8, false, false>();
    case 4: return search_fn<16, false, false>();
    case 5: return search_fn<32, false, false>();
  }
  return nullptr;
}

static size_t search_lds(int wclass, bool hbm) {
  bool lr = !hbm && mce_search_lds_rows(wclass);
  bool ls = !hbm && mce_search_lds_stack(wclass);
  return mce_search_lds_bytes(wclass, lr, ls);
}

int mce_search_max_workers(int wclass, bool hbm, int num_cu) {
  const void* fn = search_kernel(wclass, hbm);
  if (!fn) return 0;
  size_t lds = search_lds(wclass, hbm);
  if (lds > 64 * 1024) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return 0;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64, lds) != hipSuccess) return 0;
  long long total = (long long)per_cu * num_cu;
  if (total > MCE_MAX_WORKERS) total = MCE_MAX_WORKERS;
  return (int)total;
}

hipError_t mce_launch_search(int wclass, bool hbm, const SearchParams& prm, hipStream_t s) {
  const void* fn = search_kernel(wclass, hbm);
  if (!fn) return hipErrorInvalidValue;
  size_t lds = search_lds(wclass, hbm);
  SearchParams p = prm;
  void* args[] = {&p};
  // an ordinary launch: the worker list does not need every wave resident
  return hipLaunchKernel(fn, dim3(prm.nworkers), dim3(64), args, (unsigned)lds, s);
}
