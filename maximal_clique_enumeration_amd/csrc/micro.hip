// The search for small first-level subtrees: |P_root| <= 64 and |X_root| <= 64.
//
// "Parallelizing Maximal Clique Enumeration on GPUs" (arxiv 2212.01473v2):
//  - section 2.3, Algorithm 2 (Bron-Kerbosch with Tomita's pivot), section 2.4,
//    Algorithm 3 (independent first-level subtrees);
//  - section 3.4, full induced subgraph: bit rows for P u X over P;
//  - section 3.5: X = X_P u X_X, both bitsets here (X_X fits one word because
//    |X_root| <= 64), so the pivot comes from all of P u X;
//  - section 3.1: the page lets the threads of a block share one node's set
//    operations and splits work at sub-warp granularity; here the partition goes
//    down to one lane per search-tree node (the sets are single 64-bit words);
//  - section 3.3: idle workers receive branches from busy ones.
//
// MI355X mapping. One 64-lane wavefront works on one root's table (staged in
// LDS). A search-tree node is a self-contained frame of six words: P, X_P, X_X,
// C (branches left, once the pivot is known), the hash sum of R, and |R| with a
// started flag. The wave's lanes share one LIFO frame stack in HBM (structure of
// arrays, so a step's pops and pushes are coalesced). Each step:
//   1. lanes without a frame pop one from the top;
//   2. fresh frames compute their pivot (lane-private loop over the candidates);
//   3. every started frame takes one branch: a leaf is counted at once; a lane
//      that descends pushes its parent when the parent has branches left;
//   4. a pending branch request from an idle wave is answered with frames from
//      the bottom of the stack (the shallowest, largest ones).
// Every frame is a whole node of Algorithm 2, so any lane of any wave can carry
// it on: the order in which siblings are taken changes, the X set each one sees
// does not (a sibling taken earlier is in its X_P, a later one is not).
#include "mce_device.h"
#include "mce_internal.h"
#include "worklist.h"

#define MF 6            // words per frame
#define MICRO_DON 32    // frames per donation at most

template <bool CNT>
__global__ __launch_bounds__(64) void k_search_micro(MicroParams prm) {
  __shared__ u64 s_rows[2 * MCE_MICRO_MAX];
  __shared__ u64 s_xcol[MCE_MICRO_MAX];
  __shared__ u64 s_hv[MCE_MICRO_MAX];
  __shared__ u64 s_hist[MCE_MICRO_MAX + 4];

  const int lane = lane_id();
  const int wid = blockIdx.x;
  MceWl* wl = prm.wl;
  if (ld_relaxed(prm.status) & (MCE_E_HEAP | MCE_E_LIMIT)) return;
  const u64 t_start = wall_clock64();
  const u64 deadline = ld_relaxed64(prm.t_run) + prm.budget;
  for (int i = lane; i < MCE_MICRO_MAX + 4; i += MCE_WAVE) s_hist[i] = 0;
  wl_join(wl);
  __syncthreads();

  const u32 cap = (u32)prm.stack_cap;   // power of two
  const u32 cmask = cap - 1;
  u64* stk = prm.stacks + (size_t)wid * MF * cap;   // word j of slot i at stk[j * cap + i]
  u64* mail = prm.mail + (size_t)wid * prm.mail_words;

  u64 hacc = 0;   // per lane: sum of the clique hashes this lane reported
  u64 st_nodes = 0, st_br = 0, st_don = 0, st_roots = 0, st_recv = 0, st_prow = 0;
  u64 idle_ticks = 0;
  u32 max_depth_stack = 0;
  u64 st_steps = 0, st_lanes = 0;
  u32 rng = 0x9E3779B9u ^ ((u32)wid * 0x85EBCA6Bu) ^ (u32)prm.nroots;
  if (rng == 0) rng = 1;
  bool phase2 = false;
  bool req_closed = true;   // the request word starts closed and is closed again by wl_idle
  bool abort = false;
  u32 steps = 0;

  for (;;) {
    // ---------------------------------------------------------- a table and its first frames
    u64 toff = 0;
    int nfr = 0;
    if (!phase2) {
      const u32 idx = next_root(wl, (u32)prm.nroots);
      if (idx >= (u32)prm.nroots) {
        phase2 = true;
        continue;
      }
      toff = uni(prm.tab_off[idx]);
    } else {
      if (!prm.worker_list) break;
      const u64 t0 = wall_clock64();
      const int got = wl_idle(wl, wid, prm.nworkers, deadline, prm.status, rng);
      req_closed = true;
      idle_ticks += wall_clock64() - t0;
      if (!got) break;
      toff = uni(ld_relaxed64(&mail[0]));
      nfr = (int)uni((u32)ld_relaxed64(&mail[1]));
    }
    const u64* T = prm.heap + toff;
    const u64 hdr = uni(T[0]);
    const int p = (int)(u32)hdr;
    const int x = (int)(hdr >> 32);
    for (int i = lane; i < p + x; i += MCE_WAVE) s_rows[i] = T[3 + i];
    if (lane < p) {
      s_xcol[lane] = T[3 + p + x + lane];
      s_hv[lane] = T[3 + p + x + p + lane];
    }
    // lane frame
    u64 fP = 0, fX = 0, fXX = 0, fC = 0, fS = 0;
    int fK = 0;
    bool fst = false, has = false;
    if (!phase2) {
      if (lane == 0) {
        fP = p >= 64 ? ~0ull : ((1ull << p) - 1);
        fXX = x >= 64 ? ~0ull : ((1ull << x) - 1);
        fS = T[2];
        fK = 1;
        has = true;
      }
      st_roots++;
    } else {
      if (lane < nfr) {
        const u64* mf = mail + 2;
        fP = ld_relaxed64(&mf[0 * MICRO_DON + lane]);
        fX = ld_relaxed64(&mf[1 * MICRO_DON + lane]);
        fXX = ld_relaxed64(&mf[2 * MICRO_DON + lane]);
        fC = ld_relaxed64(&mf[3 * MICRO_DON + lane]);
        fS = ld_relaxed64(&mf[4 * MICRO_DON + lane]);
        const u64 m = ld_relaxed64(&mf[5 * MICRO_DON + lane]);
        fK = (int)(u32)m;
        fst = (m >> 32) != 0;
        has = true;
      }
      st_recv++;
    }
    __syncthreads();
    if (prm.worker_list && req_closed) {
      wl_open(wl, wid);
      req_closed = false;
    }
    u32 bot = 0, top = 0;   // the wave's stack holds slots [bot, top) (mod cap)

    // ---------------------------------------------------------- steps
    for (;;) {
      // this wave's request word, read now and acted on at the end of the step
      // (the load completes while the step works)
      u32 rq_raw = 0u;
      if (prm.worker_list) rq_raw = ld_relaxed(wl_req(wl, wid));
      // 1. lanes without a frame pop the newest ones
      const u64 idle = ballot(!has);
      const u32 avail = top - bot;
      if (idle && avail) {
        const u32 take = min((u32)__popcll(idle), avail);
        const u32 rank = (u32)mbcnt(idle);
        if (!has && rank < take) {
          const u32 slot = (top - 1u - rank) & cmask;
          fP = stk[0 * (size_t)cap + slot];
          fX = stk[1 * (size_t)cap + slot];
          fXX = stk[2 * (size_t)cap + slot];
          fC = stk[3 * (size_t)cap + slot];
          fS = stk[4 * (size_t)cap + slot];
          const u64 m = stk[5 * (size_t)cap + slot];
          fK = (int)(u32)m;
          fst = (m >> 32) != 0;
          has = true;
        }
        top -= take;
      }
      const u64 holding = ballot(has);
      if (holding == 0) break;   // this table's frames are all done here
      st_steps++;
      st_lanes += (u64)__popcll(holding);
      if ((++steps & 255u) == 0) {
        int stop = 0;
        if (lane == 0) {
          if (ld_relaxed(&wl->done)) {
            stop = 1;
          } else if (past_deadline(deadline)) {
            atomicOr(prm.status, MCE_E_TIMEOUT);
            st_relaxed(&wl->done, 1u);
            stop = 1;
          }
        }
        if (read_lane(stop, 0)) {
          abort = true;
          break;
        }
      }

      // 2. pivot of the fresh frames: the candidate of P u X_P u X_X with the
      //    most neighbours in P (Tomita); an X vertex adjacent to all of P ends
      //    the node at once
      const bool fresh = has && !fst;
      st_nodes += (u64)__popcll(ballot(fresh));
      if (fresh) {
        const u32 pc = (u32)__popcll(fP);
        u64 cm = fP | fX;
        u32 bc = 0;
        u64 brow = 0;
        bool found = false;
        while (cm) {
          const int u = __builtin_ctzll(cm);
          cm &= cm - 1;
          const u64 r = s_rows[u];
          const u32 c = (u32)__popcll(fP & r);
          if (!found || c > bc) {
            bc = c;
            brow = r;
            found = true;
          }
          if constexpr (CNT) st_prow++;
        }
        u64 cx = fXX;
        while (cx && bc < pc) {
          const int a = __builtin_ctzll(cx);
          cx &= cx - 1;
          const u64 r = s_rows[p + a];
          const u32 c = (u32)__popcll(fP & r);
          if (c > bc) {
            bc = c;
            brow = r;
          }
          if constexpr (CNT) st_prow++;
        }
        fC = fP & ~brow;
        fst = true;
        if (fC == 0) has = false;
      }

      // 3. one branch per started frame (Algorithm 2: child (P n N(v), X n N(v)),
      //    then P -= {v}, X += {v})
      const bool br = has && fst;
      st_br += (u64)__popcll(ballot(br));
      bool push = false, emit = false;
      int kemit = 0;
      u64 pP = 0, pX = 0, pXX = 0, pC = 0, pS = 0;
      int pK = 0;
      if (br) {
        const int v = __builtin_ctzll(fC);
        const u64 vbit = 1ull << v;
        fC ^= vbit;
        fP ^= vbit;
        const u64 r = s_rows[v];
        const u64 pn = fP & r;
        const u64 xn = fX & r;
        const u64 xxn = fXX & s_xcol[v];
        fX |= vbit;
        const u64 sc = fS + s_hv[v];
        const int kc = fK + 1;
        if (pn == 0) {
          // a leaf: R u {v} is maximal iff X n N(v) is empty
          if ((xn | xxn) == 0) {
            emit = true;
            kemit = kc;
            hacc += mce_clique_term(sc, kc);
          }
          if (fC == 0) has = false;
        } else {
          push = fC != 0;
          pP = fP;
          pX = fX;
          pXX = fXX;
          pC = fC;
          pS = fS;
          pK = fK;
          fP = pn;
          fX = xn;
          fXX = xxn;
          fS = sc;
          fK = kc;
          fst = false;
        }
      }
      const u64 em = ballot(emit);
      if (em) {
        const int kf = read_lane(kemit, __builtin_ctzll(em));
        const u64 same = ballot(emit && kemit == kf);
        if (lane == 0) atomicAdd(&s_hist[kf], (u64)__popcll(same));
        if (emit && kemit != kf) atomicAdd(&s_hist[kemit], 1ull);
      }
      // parents with branches left go on the stack
      const u64 pm = ballot(push);
      if (pm) {
        const u32 np = (u32)__popcll(pm);
        if (top - bot + np > cap) {   // the stack is sized far beyond any depth x lanes
          if (lane == 0) {
            atomicOr(prm.status, MCE_E_LIMIT);
            st_relaxed(&wl->done, 1u);
          }
          abort = true;
          break;
        }
        if (push) {
          const u32 slot = (top + (u32)mbcnt(pm)) & cmask;
          stk[0 * (size_t)cap + slot] = pP;
          stk[1 * (size_t)cap + slot] = pX;
          stk[2 * (size_t)cap + slot] = pXX;
          stk[3 * (size_t)cap + slot] = pC;
          stk[4 * (size_t)cap + slot] = pS;
          stk[5 * (size_t)cap + slot] = (u64)(u32)pK | (1ull << 32);
        }
        top += np;
        max_depth_stack = max(max_depth_stack, top - bot);
      }

      // 4. branch requests: frames from the bottom of the stack
      if (prm.worker_list) {
        const u32 rq = uni(rq_raw);
        if (rq != 0u && rq != MCE_REQ_CLOSED) {
          const int rcv = (int)rq - 1;
          // half the stack (rounded up, at most MICRO_DON frames) if the frames
          // hold at least donate_min_p candidate vertices together
          u32 give = min((top - bot + 1u) / 2u, (u32)MICRO_DON);
          const u64 gp = (u32)lane < give ? stk[0 * (size_t)cap + ((bot + (u32)lane) & cmask)] : 0ull;
          if (give && wave_sum_u32((u32)__popcll(gp)) < (u32)prm.donate_min_p) give = 0;
          if (give) {
            u64* dm = prm.mail + (size_t)rcv * prm.mail_words;
            u64* df = dm + 2;
            if ((u32)lane < give) {
              const u32 slot = (bot + (u32)lane) & cmask;
              for (int j = 0; j < MF; j++) st_relaxed64(&df[j * MICRO_DON + lane], stk[(size_t)j * cap + slot]);
            }
            if (lane == 0) {
              st_relaxed64(&dm[0], toff);
              st_relaxed64(&dm[1], (u64)give);
            }
            bot += give;
            wl_give(wl, wid, rcv);
            st_don++;
          } else {
            wl_refuse(wl, wid, rcv);
          }
        }
      }
      // Stack slots pass between lanes of this wave from step to step: the
      // vector memory operations of one wave are coherent with each other, and
      // this keeps the compiler from moving them across steps.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    if (abort) break;
  }

  // ---------------------------------------------------------- flush
  const u64 t_end = wall_clock64();
  const u64 hsum = wave_sum_u64(hacc);
  __syncthreads();
  u64 mine = 0;
  for (int i = lane; i < MCE_MICRO_MAX + 4; i += MCE_WAVE) {
    const u64 h = s_hist[i];
    mine += h;
    if (h && !abort) atomicAdd(&prm.g_hist[i], h);
  }
  const u64 leaves = wave_sum_u64(mine);
  if (!abort && lane == 0 && hsum) atomicAdd(prm.g_hash, hsum);
  const u64 prow = CNT ? wave_sum_u64(st_prow) : 0ull;
  if (lane == 0) {
    u64* st = prm.stats + (size_t)wid * MCE_NSTAT;
    const u64 total = t_end - t_start;
    st[ST_NODES] = st_nodes;
    st[ST_LEAVES] = leaves;
    st[ST_DONATIONS] = st_don;
    st[ST_PIVOT_ROWS] = prow;
    st[ST_PIVOT_WORDS] = prow;
    st[ST_XX_TESTS] = 0;
    st[ST_BRANCHES] = st_br;
    st[ST_BUSY_TICKS] = total - idle_ticks;
    st[ST_ROOTS] = st_roots;
    st[ST_RECEIVED] = st_recv;
    st[ST_TOTAL_TICKS] = total;
    st[ST_START_ABS] = t_start;
    st[ST_STACK_MAX] = max_depth_stack;
    st[ST_STEPS] = st_steps;
    st[ST_LANE_STEPS] = st_lanes;
  }
}

// ------------------------------------------------------------------ host side
static const void* micro_kernel(bool counters) {
  return counters ? (const void*)k_search_micro<true> : (const void*)k_search_micro<false>;
}

int mce_micro_mail_words() { return 2 + MF * MICRO_DON; }

int mce_micro_max_workers(bool counters, int num_cu) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, micro_kernel(counters), 64, 0) != hipSuccess) return 0;
  long long total = (long long)per_cu * num_cu;
  if (total > MCE_MAX_WORKERS) total = MCE_MAX_WORKERS;
  return (int)total;
}

hipError_t mce_launch_micro(bool counters, const MicroParams& prm, hipStream_t s) {
  MicroParams p = prm;
  void* args[] = {&p};
  return hipLaunchKernel(micro_kernel(counters), dim3(prm.nworkers), dim3(64), args, 0, s);
}
