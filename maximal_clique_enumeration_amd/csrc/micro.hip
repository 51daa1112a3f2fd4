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
// C (branches left, once the pivot is known), the hash sum of R, and |R|. The
// wave's lanes share one LIFO stack of started frames (pivot known, branches
// left): its top MICRO_L frames live in LDS, older ones spill to a per-wave HBM
// area (structure of arrays, so spills and refills are coalesced). Each step:
//   1. lanes without a frame pop the newest ones;
//   2. lanes whose frame has no pivot yet score up to MICRO_K pivot candidates
//      (Tomita: the vertex of P u X with the most neighbours in P); a frame with
//      more candidates carries its partial maximum into the next step, so one
//      shallow frame does not hold 63 lanes for a whole scan. In launches of
//      many small roots, a step where few lanes need a pivot and one of them has
//      many candidates left shares the scans out over lane groups (coop_pivot);
//   3. lanes with a started frame take branches: up to MICRO_B leaf branches
//      (R u {v} with P n N(v) empty) in a row, or one branch that descends, after
//      which the parent goes on the stack if it has branches left;
//   4. a pending branch request from an idle wave is answered with frames from
//      the bottom of the stack (the shallowest, largest ones).
// Every frame is a whole node of Algorithm 2, so any lane of any wave can carry
// it on: the order in which siblings are taken changes, the X set each one sees
// does not (a sibling taken earlier is in its X_P, a later one is not).
#include "mce_device.h"
#include "mce_internal.h"
#include "worklist.h"

#ifndef MICRO_K
#define MICRO_K 8      // pivot candidates scored per lane and step
#endif
#ifndef MICRO_B
#define MICRO_B 4      // leaf branches per lane and step
#endif
#ifndef MICRO_L
#define MICRO_L 256    // stack frames kept in LDS (power of two, >= 128)
#endif
#define MF 6           // words per frame
#define MICRO_QCAP (MCE_WAVE * (MICRO_B + 1))
#define MICRO_DON 32   // frames per donation at most

#ifndef MICRO_CQ
#define MICRO_CQ 4     // pivot scans shared out over lane groups when at most this many lanes need one
#endif
#ifndef MICRO_CQ_MIN
#define MICRO_CQ_MIN (2 * MICRO_K)   // ... and one of them has more candidates left than this
#endif

static_assert((MICRO_L & (MICRO_L - 1)) == 0 && MICRO_L >= 128, "LDS stack size");
static_assert(MICRO_CQ == 1 || MICRO_CQ == 2 || MICRO_CQ == 4 || MICRO_CQ == 8 || MICRO_CQ == 16,
              "cooperative scan bound");

// Lane value exchange through the LDS crossbar (every lane active).
__device__ __forceinline__ u32 lane_fetch(u32 v, int src) {
  return (u32)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}
__device__ __forceinline__ u64 lane_fetch(u64 v, int src) {
  return ((u64)lane_fetch((u32)(v >> 32), src) << 32) | lane_fetch((u32)v, src);
}

// Cooperative pivot scan, for a step in which at most 64 / GL lanes need one:
// group g (lanes g GL .. g GL + GL - 1) scores every remaining candidate of the
// g-th such lane's frame, lane s of the group the candidates at bit positions
// s, s + GL, s + 2 GL, ... of its P u X_P and X_X candidate masks, and the
// group's maximum goes back to the frame's lane with its row. The whole scan
// ends in this step, where one lane alone scores MICRO_K candidates per step.
// Any maximiser of |P n N(u)| is a valid pivot (section 2.3), so the
// tie-break (highest lane) does not change the cliques found. Every lane
// active; pvm, xx uniform.
template <int GL>
__device__ __forceinline__ void coop_pivot(const u64* s_rows, int lane, u64 pvm, bool xx, bool pv, u64 fP,
                                           u64& pcm, u64& pcx, u32& pbc, u64& pbr, u64& nrows) {
  constexpr int NG = MCE_WAVE / GL;   // groups, and bit positions per lane
  const int grp = lane / GL, sub = lane % GL;
  u64 m = pvm;
  int own = MCE_WAVE;   // none: the group has no frame to score
#pragma unroll
  for (int t = 0; t < NG; t++) {
    const int o = m ? __builtin_ctzll(m) : MCE_WAVE;
    own = t == grp ? o : own;
    m &= m - 1ull;
  }
  // (the fetches run in every lane: a permute reads nothing from a lane that is
  // switched off, and a frame's lane may sit in a group without a frame)
  const int src = own < MCE_WAVE ? own : lane;
  const u64 oP = lane_fetch(fP, src);
  const u64 fM = lane_fetch(pcm, src);
  const u64 fX = xx ? lane_fetch(pcx, src) : 0ull;
  const u64 oM = own < MCE_WAVE ? fM : 0ull;
  const u64 oX = own < MCE_WAVE ? fX : 0ull;
  u64 rr[NG];
#pragma unroll
  for (int j = 0; j < NG; j++) rr[j] = s_rows[sub + j * GL];
  u32 best = 0;
  u64 brow = 0;
#pragma unroll
  for (int j = 0; j < NG; j++) {
    const u32 c = (oM >> (sub + j * GL)) & 1ull ? (u32)__popcll(oP & rr[j]) + 1u : 0u;
    if (c > best) {
      best = c;
      brow = rr[j];
    }
  }
  if (xx) {
#pragma unroll
    for (int j = 0; j < NG; j++) rr[j] = s_rows[MCE_MICRO_MAX + sub + j * GL];
#pragma unroll
    for (int j = 0; j < NG; j++) {
      const u32 c = (oX >> (sub + j * GL)) & 1ull ? (u32)__popcll(oP & rr[j]) + 1u : 0u;
      if (c > best) {
        best = c;
        brow = rr[j];
      }
    }
  }
  // group maximum of (score, lane); then the frame's lane takes it from lane g GL
  u32 key = (best << 8) | (u32)lane;
#pragma unroll
  for (int off = GL / 2; off >= 1; off >>= 1) {
    const u32 o = lane_fetch(key, lane ^ off);
    key = o > key ? o : key;
  }
  const int r = mbcnt(pvm);
  const u32 k2 = lane_fetch(key, pv ? r * GL : lane);
  const u64 row = lane_fetch(brow, (int)(k2 & 63u));
  if (pv) {
    nrows += (u64)(__popcll(pcm) + __popcll(pcx));
    if ((k2 >> 8) > pbc) {
      pbc = k2 >> 8;
      pbr = row;
    }
    pcm = 0ull;
    pcx = 0ull;
  }
}

// COOP: the kernel instance with cooperative pivot scans (launches of many
// small roots). It is a separate instance because the extra code alone makes
// the compiler lay out the step loop of the other one worse (4-8 % slower).
template <bool CNT, bool COOP>
__global__ __launch_bounds__(64) void k_search_micro(MicroParams prm) {
  __shared__ u64 s_rows[2 * MCE_MICRO_MAX];
  __shared__ u64 s_xcol[MCE_MICRO_MAX];
  __shared__ u64 s_hv[MCE_MICRO_MAX];
  __shared__ u64 s_hist[MCE_MICRO_MAX + 4];
  __shared__ u64 s_stk[MF][MICRO_L];
  // found cliques waiting for their hash mix (sum of member terms + |C| G),
  // mixed 64 at a time so that every lane of the mix is busy
  __shared__ u64 s_q[MICRO_QCAP];

  const int lane = lane_id();
  const int wid = blockIdx.x;
  MceWl* wl = prm.wl;
  // a failed build, or a run already past its time limit: search nothing
  if (ld_relaxed(prm.status) & MCE_E_STOP) {
    if (wid == 0 && lane == 0 && prm.taken) {
      const u32 ctr = ld_relaxed(&wl->root_ctr);
      st_relaxed(prm.taken, min(ctr, (u32)prm.nroots));
    }
    return;
  }
  const u64 t_start = wall_clock64();
  const u64 hwloc = wave_hw_location();
  ActClock<CNT> act;   // per-activity cycles (counting instance)
  act.start();
  const u64 deadline = ld_relaxed64(prm.t_run) + prm.budget;
  for (int i = lane; i < MCE_MICRO_MAX + 4; i += MCE_WAVE) s_hist[i] = 0;
  wl_join(wl);
  __syncthreads();

  const u32 cap = (u32)prm.stack_cap;   // HBM frames per wave, a power of two
  const u32 cmask = cap - 1u;
  const u32 lmask = MICRO_L - 1u;
  u64* hstk = prm.stacks + (size_t)wid * MF * cap;   // word j of slot i at hstk[j * cap + i]
  u64* mail = prm.mail + (size_t)wid * prm.mail_words;

  u64 hacc = 0;   // per lane: sum of the clique hashes this lane mixed
  u32 qn = 0;     // cliques in s_q (uniform)
  u64 st_nodes = 0, st_br = 0, st_don = 0, st_roots = 0, st_recv = 0, st_prow = 0;
  u64 st_steps = 0, st_lanes = 0;
  u64 idle_ticks = 0;
  u32 max_stack = 0;
  u32 rng = 0x9E3779B9u ^ ((u32)wid * 0x85EBCA6Bu) ^ (u32)prm.nroots;
  if (rng == 0) rng = 1;
  u64 t_first = 0, t_last = 0;
  bool phase2 = false;
  bool req_closed = true;   // the request word starts closed and is closed again by wl_idle
  bool abort = false;
  u32 steps = 0;
  RootCursor rc{0u, 0u};

  for (;;) {
    // ---------------------------------------------------------- a table and its first frames
    u64 toff = 0;
    int nfr = 0;
    if (!phase2) {
      const u32 idx = take_root(wl, rc, (u32)prm.nroots, (u32)prm.nworkers, 64u);
      act.mark(ACT_WL);
      if (idx >= (u32)prm.nroots) {
        phase2 = true;
        continue;
      }
      toff = uni(prm.tab_off[idx]) - uni(prm.tab_off[0]);
    } else {
      if (!prm.worker_list) break;
      const u64 t0 = wall_clock64();
      const int got = wl_idle(wl, wid, prm.nworkers, deadline, prm.status, rng, MCE_REQ_SLOTS);
      act.mark(ACT_IDLE);
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
    // rows: P member j at j, X_X member a at MCE_MICRO_MAX + a
    if (lane < p) s_rows[lane] = T[3 + lane];
    if (lane < x) s_rows[MCE_MICRO_MAX + lane] = T[3 + p + lane];
    if (lane < p) {
      s_xcol[lane] = T[3 + p + x + lane];
      s_hv[lane] = T[3 + p + x + p + lane];
    }
    // the lane's frame, and its pivot scan while the frame is not started
    u64 fP = 0, fX = 0, fXX = 0, fC = 0, fS = 0;
    int fK = 0;
    bool fst = false, has = false;
    u64 pcm = 0, pcx = 0;   // candidates left to score: P u X_P rows, X_X rows
    u32 pbc = 0;            // best score so far: neighbours in P plus one (0: none yet)
    u64 pbr = 0;            // its row
    if (!phase2) {
      if (lane == 0) {
        fP = p >= 64 ? ~0ull : ((1ull << p) - 1);
        fXX = x >= 64 ? ~0ull : ((1ull << x) - 1);
        fS = T[2];
        fK = (int)(T[1] >> 32);   // |R| at the root
        has = true;
        pcm = fP;
        pcx = fXX;
      }
      st_roots++;
    } else {
      if (lane < nfr) {   // donated frames are started
        const u64* mf = mail + 2;
        fP = ld_relaxed64(&mf[0 * MICRO_DON + lane]);
        fX = ld_relaxed64(&mf[1 * MICRO_DON + lane]);
        fXX = ld_relaxed64(&mf[2 * MICRO_DON + lane]);
        fC = ld_relaxed64(&mf[3 * MICRO_DON + lane]);
        fS = ld_relaxed64(&mf[4 * MICRO_DON + lane]);
        fK = (int)ld_relaxed64(&mf[5 * MICRO_DON + lane]);
        fst = true;
        has = true;
      }
      st_recv++;
    }
    __syncthreads();
    if (prm.worker_list && req_closed) {
      wl_open(wl, wid, MCE_REQ_SLOTS);
      req_closed = false;
    }
    if (t_first == 0) t_first = wall_clock64();
    act.mark(ACT_STAGE);
    // the stack holds virtual slots [bot, top): [bot, mid) in HBM (slot & cmask),
    // [mid, top) in LDS (slot & lmask)
    u32 bot = 0, mid = 0, top = 0;

    // ---------------------------------------------------------- steps
    for (;;) {
      // this wave's request word, read now and acted on at the end of the step
      u32 rq_raw = 0u;
      if (prm.worker_list && lane < MCE_REQ_SLOTS) rq_raw = ld_relaxed(wl_req(wl, wid, lane));

      // 1. lanes without a frame pop the newest ones
      const u64 idle = ballot(!has);
      if (idle && top != bot) {
        if (top == mid) {
          // LDS part empty: bring the newest HBM frames back
          const u32 f = min(mid - bot, (u32)MCE_WAVE);
          if ((u32)lane < f) {
            const u32 v = mid - f + (u32)lane;
            for (int j = 0; j < MF; j++) s_stk[j][v & lmask] = hstk[(size_t)j * cap + (v & cmask)];
          }
          mid -= f;
          __syncthreads();
        }
        const u32 take = min((u32)__popcll(idle), top - mid);
        const u32 rank = (u32)mbcnt(idle);
        if (!has && rank < take) {
          const u32 sl = (top - 1u - rank) & lmask;
          fP = s_stk[0][sl];
          fX = s_stk[1][sl];
          fXX = s_stk[2][sl];
          fC = s_stk[3][sl];
          fS = s_stk[4][sl];
          fK = (int)s_stk[5][sl];
          fst = true;
          has = true;
        }
        top -= take;
      }
      const u64 holding = ballot(has);
      act.mark(ACT_STACK);
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

      // 2. pivot scan (Tomita): score the next MICRO_K candidates of P u X_P
      //    (rows 0..p-1) and X_X (rows from MCE_MICRO_MAX) by |P n N(u)|; the
      //    candidates are picked first so that their row reads overlap. An X
      //    vertex adjacent to all of P ends the node (no maximal clique below it).
      const bool pv = has && !fst;
      const u64 pvm = ballot(pv);
      if (pvm) {
        const u32 pc1 = (u32)__popcll(fP) + 1u;   // a score of pc1 means |P n N(u)| = |P|
        const bool xx = ballot(pv && pcx != 0ull) != 0ull;
        // few frames to score, one of them with more than MICRO_CQ_MIN
        // candidates left: the lanes share the scans out (coop_pivot)
        bool coop = false;
        if constexpr (COOP) {
          const int q = __popcll(pvm);
          if (q <= MICRO_CQ &&
              wave_max_u32(pv ? (u32)(__popcll(pcm) + __popcll(pcx)) : 0u) > (u32)MICRO_CQ_MIN) {
            coop = true;
            u64 crows = 0;
            if (q <= 1) {
              coop_pivot<64>(s_rows, lane, pvm, xx, pv, fP, pcm, pcx, pbc, pbr, crows);
            } else if (MICRO_CQ >= 2 && q <= 2) {
              coop_pivot<32>(s_rows, lane, pvm, xx, pv, fP, pcm, pcx, pbc, pbr, crows);
            } else if (MICRO_CQ >= 4 && q <= 4) {
              coop_pivot<16>(s_rows, lane, pvm, xx, pv, fP, pcm, pcx, pbc, pbr, crows);
            } else if (MICRO_CQ >= 8 && q <= 8) {
              coop_pivot<8>(s_rows, lane, pvm, xx, pv, fP, pcm, pcx, pbc, pbr, crows);
            } else {
              coop_pivot<4>(s_rows, lane, pvm, xx, pv, fP, pcm, pcx, pbc, pbr, crows);
            }
            if constexpr (CNT) st_prow += crows;
          }
        }
        if (!coop && pv) {
          {
            int cu[MICRO_K];
            bool cv[MICRO_K];
            if (xx) {
#pragma unroll
              for (int i = 0; i < MICRO_K; i++) {
                cv[i] = (pcm | pcx) != 0ull;
                if (pcm) {
                  cu[i] = __builtin_ctzll(pcm);
                  pcm &= pcm - 1ull;
                } else if (pcx) {
                  cu[i] = MCE_MICRO_MAX + __builtin_ctzll(pcx);
                  pcx &= pcx - 1ull;
                } else {
                  cu[i] = 0;
                }
              }
            } else {   // no X_X candidate in any lane
#pragma unroll
              for (int i = 0; i < MICRO_K; i++) {
                cv[i] = pcm != 0ull;
                cu[i] = cv[i] ? __builtin_ctzll(pcm) : 0;
                pcm &= pcm - 1ull;
              }
            }
            u64 cr[MICRO_K];
#pragma unroll
            for (int i = 0; i < MICRO_K; i++) cr[i] = s_rows[cu[i]];
#pragma unroll
            for (int i = 0; i < MICRO_K; i++) {
              const u32 c = cv[i] ? (u32)__popcll(fP & cr[i]) + 1u : 0u;
              if (c > pbc) {
                pbc = c;
                pbr = cr[i];
              }
              if constexpr (CNT) st_prow += cv[i] ? 1u : 0u;
            }
          }
        }
        const bool done = pv && ((pcm | pcx) == 0ull || pbc >= pc1);
        st_nodes += (u64)__popcll(ballot(done));
        if (done) {
          fC = pbc >= pc1 ? 0ull : fP & ~pbr;
          fst = true;
          if (fC == 0) has = false;
        }
      }

      act.mark(ACT_PIVOT);
      // 3. branches (Algorithm 2: child (P n N(v), X n N(v)), then P -= {v},
      //    X += {v}) in ascending order of v; the next MICRO_B branch vertices are
      //    known up front, so their reads overlap. Leaf branches are taken in a
      //    row; a descending one ends the lane's step.
      bool push = false;
      u32 nemit = 0;
      int kemit = 0;
      u64 pP = 0, pX = 0, pXX = 0, pC = 0, pS = 0;
      int pK = 0;
      // (the loop runs in every lane so that found cliques can be queued with
      // wave-wide ballots; lanes without a started frame take no branch)
      {
        const bool brl = has && fst;
        int bv[MICRO_B];
        bool bval[MICRO_B];
        u64 cm = brl ? fC : 0ull;
#pragma unroll
        for (int i = 0; i < MICRO_B; i++) {
          bval[i] = cm != 0ull;
          bv[i] = bval[i] ? __builtin_ctzll(cm) : 0;
          cm &= cm - 1ull;
        }
        u64 br_row[MICRO_B], br_xc[MICRO_B], br_hv[MICRO_B];
#pragma unroll
        for (int i = 0; i < MICRO_B; i++) {
          br_row[i] = s_rows[bv[i]];
          br_xc[i] = s_xcol[bv[i]];
          br_hv[i] = s_hv[bv[i]];
        }
        bool go = brl;
#pragma unroll
        for (int i = 0; i < MICRO_B; i++) {
          bool emit = false;
          u64 z = 0;
          if (go && bval[i]) {
            const u64 vbit = 1ull << bv[i];
            fC ^= vbit;
            fP ^= vbit;
            const u64 r = br_row[i];
            const u64 pn = fP & r;
            const u64 xn = fX & r;
            const u64 xxn = fXX & br_xc[i];
            fX |= vbit;
            const u64 sc = fS + br_hv[i];
            const int kc = fK + 1;
            if constexpr (CNT) st_br++;
            if (pn == 0) {
              // a leaf: R u {v} is maximal iff X n N(v) is empty
              if ((xn | xxn) == 0) {
                nemit++;
                kemit = kc;
                emit = true;
                z = sc + (u64)kc * MCE_GOLDEN;
              }
              if (fC == 0) {
                has = false;
                go = false;
              }
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
              pcm = pn | xn;
              pcx = xxn;
              pbc = 0;
              go = false;
            }
          }
          const u64 qm = ballot(emit);
          if (qm) {
            if (emit) s_q[qn + (u32)mbcnt(qm)] = z;
            qn += (u32)__popcll(qm);
          }
        }
      }
      act.mark(ACT_SETOPS);
      // a full round of queued cliques: mix one per lane
      while (qn >= (u32)MCE_WAVE) {
        qn -= (u32)MCE_WAVE;
        hacc += mce_mix64(s_q[qn + (u32)lane]);
      }
      // clique sizes: one shared counter update for the most common size
      const u64 em = ballot(nemit != 0);
      if (em) {
        const int kf = read_lane(kemit, __builtin_ctzll(em));
        const bool same = nemit != 0 && kemit == kf;
        const u32 tot = wave_sum_u32(same ? nemit : 0u);
        if (lane == 0) atomicAdd(&s_hist[kf], (u64)tot);
        if (nemit != 0 && !same) atomicAdd(&s_hist[kemit], (u64)nemit);
      }
      act.mark(ACT_EMIT);
      // parents with branches left go on the stack (LDS; its oldest frames spill to HBM)
      const u64 pm = ballot(push);
      if (pm) {
        const u32 np = (u32)__popcll(pm);
        if (top - mid + np > (u32)MICRO_L) {
          // move the oldest MCE_WAVE LDS frames to HBM (top - mid > MICRO_L - 64 here)
          if (mid - bot + (u32)MCE_WAVE > cap) {
            if (lane == 0) {
              atomicOr(prm.status, MCE_E_MSTACK);
              st_relaxed(&wl->done, 1u);
            }
            abort = true;
            break;
          }
          const u32 v = mid + (u32)lane;
          for (int j = 0; j < MF; j++) hstk[(size_t)j * cap + (v & cmask)] = s_stk[j][v & lmask];
          mid += (u32)MCE_WAVE;
          __syncthreads();
        }
        if (push) {
          const u32 sl = (top + (u32)mbcnt(pm)) & lmask;
          s_stk[0][sl] = pP;
          s_stk[1][sl] = pX;
          s_stk[2][sl] = pXX;
          s_stk[3][sl] = pC;
          s_stk[4][sl] = pS;
          s_stk[5][sl] = (u64)(u32)pK;
        }
        top += np;
        max_stack = max(max_stack, top - bot);
      }

      act.mark(ACT_STACK);
      // 4. branch requests (up to MCE_REQ_SLOTS per step; slot k was read by
      //    lane k): each receiver gets an equal share of the stack's bottom
      //    frames (the shallowest), at most MICRO_DON, leaving this wave as much
      //    as one receiver, if the frames hold at least donate_min_p candidate
      //    vertices together. All mailboxes are published with one wait.
      if (prm.worker_list) {
        const bool pend = lane < MCE_REQ_SLOTS && rq_raw != 0u && rq_raw != MCE_REQ_CLOSED;
        const u64 pm = ballot(pend);
        if (pm) {
          const u32 nreq = (u32)__popcll(pm);
          const u32 share = min((u32)MICRO_DON, max(1u, (top - bot) / (nreq + 1u)));
          u64 given = 0;
          for (u64 rest = pm; rest; rest &= rest - 1ull) {
            const int k = __builtin_ctzll(rest);
            const int rcv = (int)read_lane((int)rq_raw, k) - 1;
            u32 give = min(share, top - bot);
            const u32 inh = mid - bot;   // frames in HBM
            const u32 v = bot + (u32)lane;
            u64 g[MF] = {0, 0, 0, 0, 0, 0};
            if ((u32)lane < give) {
              if ((u32)lane < inh) {
                for (int j = 0; j < MF; j++) g[j] = hstk[(size_t)j * cap + (v & cmask)];
              } else {
                for (int j = 0; j < MF; j++) g[j] = s_stk[j][v & lmask];
              }
            }
            if (give && wave_sum_u32((u32)__popcll(g[0])) < (u32)prm.donate_min_p) give = 0;
            if (!give) continue;
            u64* dm = prm.mail + (size_t)rcv * prm.mail_words;
            u64* df = dm + 2;
            if ((u32)lane < give) {
              for (int j = 0; j < MF; j++) st_relaxed64(&df[j * MICRO_DON + lane], g[j]);
            }
            if (lane == 0) {
              st_relaxed64(&dm[0], toff);
              st_relaxed64(&dm[1], (u64)give);
            }
            bot += give;
            if (give > inh) mid = bot;
            given |= 1ull << k;
          }
          // count the receivers active before they can run (see wl_give), then wake them
          if (given) {
            if (lane == 0)
              __hip_atomic_fetch_add(&wl->n_active, __popcll(given), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_stores_complete();
            st_don += (u64)__popcll(given);
          }
          if (pend) {
            st_relaxed(wl_flag(wl, (int)rq_raw - 1), ((given >> lane) & 1ull) ? MCE_FLAG_TASK : MCE_FLAG_RETRY);
            st_relaxed(wl_req(wl, wid, lane), 0u);
          }
        }
      }
      act.mark(ACT_WL);
      // Stack slots pass between lanes of this wave from step to step: the
      // vector memory and LDS operations of one wave are performed in order,
      // and this keeps the compiler from moving them across steps.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    t_last = wall_clock64();
    if (abort) break;
  }

  // ---------------------------------------------------------- flush
  // (also after a stop at the time limit: the cliques found so far are
  // reported, and the run is marked incomplete)
  if ((u32)lane < qn) hacc += mce_mix64(s_q[lane]);
  const u64 t_end = wall_clock64();
  const u64 hsum = wave_sum_u64(hacc);
  __syncthreads();
  u64 mine = 0;
  for (int i = lane; i < MCE_MICRO_MAX + 4; i += MCE_WAVE) {
    const u64 h = s_hist[i];
    mine += h;
    if (h) atomicAdd(&prm.g_hist[i], h);
  }
  const u64 leaves = wave_sum_u64(mine);
  if (lane == 0 && hsum) atomicAdd(prm.g_hash, hsum);
  if (wid == 0 && lane == 0) record_taken(prm.taken, wl, (u32)prm.nroots);
  act.mark(ACT_EMIT);
  const u64 prow = CNT ? wave_sum_u64(st_prow) : 0ull;
  const u64 nbr = CNT ? wave_sum_u64(st_br) : 0ull;
  if (lane == 0) {
    u64* st = prm.stats + (size_t)wid * MCE_NSTAT;
    const u64 total = t_end - t_start;
    st[ST_NODES] = st_nodes;
    st[ST_LEAVES] = leaves;
    st[ST_DONATIONS] = st_don;
    st[ST_PIVOT_ROWS] = prow;
    st[ST_PIVOT_WORDS] = prow;
    st[ST_XX_TESTS] = 0;
    st[ST_BRANCHES] = nbr;
    st[ST_BUSY_TICKS] = total - idle_ticks;
    st[ST_ROOTS] = st_roots;
    st[ST_RECEIVED] = st_recv;
    st[ST_TOTAL_TICKS] = total;
    st[ST_START_ABS] = t_start;
    st[ST_STACK_MAX] = max_stack;
    st[ST_STEPS] = st_steps;
    st[ST_LANE_STEPS] = st_lanes;
    st[ST_FIRST_ABS] = t_first;
    st[ST_LAST_ABS] = t_last;
    st[ST_HWID] = hwloc;
    act.store(st);
  }
}

// ------------------------------------------------------------------ host side
static const void* micro_kernel(bool counters, bool coop) {
  if (coop) return counters ? (const void*)k_search_micro<true, true> : (const void*)k_search_micro<false, true>;
  return counters ? (const void*)k_search_micro<true, false> : (const void*)k_search_micro<false, false>;
}

int mce_micro_mail_words() { return 2 + MF * MICRO_DON; }

int mce_micro_max_workers(bool counters, int num_cu) {
  int per_cu = 0, per_cu_coop = 0;   // both instances: the launch picks one after sizing
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, micro_kernel(counters, false), 64, 0) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_coop, micro_kernel(counters, true), 64, 0) != hipSuccess)
    return 0;
  long long total = (long long)std::min(per_cu, per_cu_coop) * num_cu;
  if (total > MCE_MAX_WORKERS) total = MCE_MAX_WORKERS;
  return (int)total;
}

hipError_t mce_launch_micro(bool counters, const MicroParams& prm, hipStream_t s) {
  MicroParams p = prm;
  void* args[] = {&p};
  return hipLaunchKernel(micro_kernel(counters, prm.coop != 0), dim3(prm.nworkers), dim3(64), args, 0, s);
}
