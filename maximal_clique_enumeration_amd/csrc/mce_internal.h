// Internal interface between the engine (host) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "mce_device.h"

struct SubOffsets {
  int off[MCE_NSUB];
};

// Activities of the per-activity cycle breakdown ("Parallelizing Maximal Clique
// Enumeration on GPUs", section 4.5 and Figure 5, which counts cycles per block
// and activity with clock reads). The build kernels are timed per launch.
enum {
  ACT_WL = 0,    // worker-list operations: taking subtrees, answering requests, handing branches over
  ACT_IDLE,      // no task: waiting for one (asking busy waves for branches) until the launch ends
  ACT_STAGE,     // a task's start: its induced subgraph and mailbox read into registers and LDS
  ACT_PIVOT,     // Tomita pivot selection
  ACT_SETOPS,    // the branches' set operations: P n N(v), X n N(v), the X_X filter, leaf tests
  ACT_STACK,     // the DFS stack: pushes, pops, spills and refills
  ACT_EMIT,      // found cliques: hash terms mixed, size histogram
  MCE_NACT
};

// Per-wavefront statistics written by the search kernel (u64 each).
enum {
  ST_NODES = 0,
  ST_LEAVES,
  ST_DONATIONS,
  ST_PIVOT_ROWS,
  ST_PIVOT_WORDS,
  ST_XX_TESTS,
  ST_BRANCHES,       // branches taken (child nodes and leaf tests)
  ST_BUSY_TICKS,
  ST_ROOTS,
  ST_RECEIVED,
  ST_TOTAL_TICKS,
  ST_DONATE_TICKS,   // handing branches over (claim + mailbox + wake)
  ST_SETUP_TICKS,    // receiving: mailbox and induced subgraph read until the search starts
  ST_FIRST_TICKS,    // kernel start until the first task (root or received) starts
  ST_START_ABS,      // wall-clock tick at which the wave started
  ST_CHECKS,         // worker-list claim attempts
  ST_DONATE_OK_TICKS,  // ticks of the successful donations alone
  ST_STACK_MAX,      // micro kernel: most frames the wave's stack held
  ST_STEPS,          // micro kernel: steps (every lane advances its frame by one node or branch)
  ST_LANE_STEPS,     // micro kernel: lanes holding a frame, summed over steps
  ST_FIRST_ABS,      // wall-clock tick at which the first task started (0: none)
  ST_LAST_ABS,       // wall-clock tick at which the last task ended
  ST_HWID,           // where the wave ran: XCC_ID << 32 | HW_ID (compute unit, shader array, engine)
  ST_ACT0,           // counting instances: shader-clock cycles per activity (MCE_NACT words)
  MCE_NSTAT = ST_ACT0 + MCE_NACT
};

// Where a wave runs: XCC_ID (bits 3:0 of HW_REG_XCC_ID: the accelerator
// complex die) in the high word, HW_REG_HW_ID in the low word (wave slot,
// SIMD, compute unit in bits 11:8, shader array bit 12, shader engine bits
// 15:13). The compute unit a wave ran on is (XCC_ID, bits 15:8 of HW_ID).
__device__ __forceinline__ u64 wave_hw_location() {
  const u32 hw = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));    // hwreg(HW_REG_HW_ID)
  const u32 xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11));  // hwreg(HW_REG_XCC_ID, 0, 16)
  return ((u64)(xcc & 0xFu) << 32) | hw;
}

// The end of a search launch, by wave 0 as it leaves: the subtrees handed out
// (every one when the launch was not stopped; otherwise those taken from the
// counter by then, each finished or abandoned at the stop).
__device__ __forceinline__ void record_taken(u32* taken, const MceWl* wl, u32 nroots) {
  if (!taken) return;
  const u32 stopped = __hip_atomic_load(&wl->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u32 ctr = __hip_atomic_load(&wl->root_ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(taken, stopped ? (ctr < nroots ? ctr : nroots) : nroots, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Cycle accounting of the counting kernel instances: each mark charges the
// cycles since the previous mark to one activity, so the activities of a wave
// add up to its whole run. ON = false compiles to nothing.
template <bool ON>
struct ActClock {
  u64 t = 0;
  u64 c[MCE_NACT] = {};
  __device__ __forceinline__ void start() {
    if constexpr (ON) t = (u64)clock64();
  }
  __device__ __forceinline__ void mark(int a) {
    if constexpr (ON) {
      const u64 n = (u64)clock64();
      c[a] += n - t;
      t = n;
    }
  }
  __device__ __forceinline__ void store(u64* st) const {
    if constexpr (ON) {
#pragma unroll
      for (int i = 0; i < MCE_NACT; i++) st[ST_ACT0 + i] = c[i];
    }
  }
};

// Where one search launch keeps its per-wave state: LDS word offsets (dynamic
// shared memory) and byte offsets inside the wave's HBM slot.
struct SearchLayout {
  int sub, wclass, mode;
  int pcap, xcap, rcap;   // largest |P|, |X|, row count over the launch's roots
  int levels, hcap;       // stack records, histogram entries
  bool srows, sstack;     // rows + X_X staged in LDS; level stack in LDS
  bool sprows;            // (without srows) the P rows staged in LDS
  bool counters;          // count pivot rows and X_X tests (width 1 keeps them out of the timed kernel)
  int l_misc, l_hist, l_hv, l_pid, l_stack, l_rows, l_xx;
  size_t lds_bytes;
  size_t s_stack, s_xx, s_mail, slot_bytes;
};

struct SearchParams {
  const int* rp;
  const int* ci;
  const u64* heap;       // induced-subgraph tables of this launch's roots
  const u64* tab_off;    // table offset of each root (by list index), relative to tab_off[0]
  int nroots;
  int nworkers;
  int hcap;
  int l_misc, l_hist, l_hv, l_pid, l_stack, l_rows, l_xx;
  size_t slot_bytes, s_stack, s_xx, s_mail;
  u64* g_hist;           // global histogram (MCE_MAX_P + 2 entries)
  u64* g_hash;
  MceWl* wl;
  char* slots;           // one HBM slot per wavefront
  int donate_min_p;
  int worker_list;
  u64 budget;            // wall-clock ticks after the run start (t_run) at which the search is abandoned
  const u64* t_run;      // run start tick, written by the peel
  u32* status;
  u64* stats;            // nworkers * MCE_NSTAT
  u32* taken;            // wave 0 stores, as it leaves, the subtrees this launch handed out
};

// The micro search (|P| <= 64, |X| <= 64): one frame per lane, a frame stack
// per wavefront in HBM (structure of arrays: word j of slot i at j * cap + i).
struct MicroParams {
  const u64* heap;
  const u64* tab_off;    // relative to tab_off[0], as in SearchParams
  int nroots;
  int nworkers;
  u64* stacks;           // nworkers * 6 * stack_cap words
  int stack_cap;         // frames per wave, a power of two
  int mail_words;        // u64 words of one mailbox
  u64* mail;             // nworkers mailboxes
  u64* g_hist;
  u64* g_hash;
  MceWl* wl;
  int donate_min_p;
  int worker_list;
  int coop;              // share pivot scans out over lane groups (many more roots than waves)
  u64 budget;
  const u64* t_run;
  u32* status;
  u64* stats;            // nworkers * MCE_NSTAT
  u32* taken;            // as in SearchParams
};

struct BuildParams {
  const int* rp;
  const int* ci;
  const int* rnd;
  const int* roots;      // the sub-class's roots
  int nroots;
  int W;                 // bitset words of the sub-class
  int mode;              // MCE_MODE_IP / MCE_MODE_IPX
  int micro;             // micro table: full rows plus the X column of every P member
  int parts;             // > 0: split build, each root's 64-row slabs dealt over this many blocks
  int l2;                // roots are CSR entries (v_i, v_j): second-level subtrees (section 3.2)
  const int* src;        // second-level roots: the COO source of every CSR entry
  u64* heap;
  u64 heap_words;
  const u64* tab_off;    // each root's table offset, as an exclusive prefix sum of table sizes that
                         // runs over all sub-classes: offsets relative to tab_off[0]
  u32* status;
  const int* hub_id;     // second-level subtrees: hub index of each vertex (-1: none), or NULL
  const u64* hub_bm;     // hub adjacency bitmaps, hub_words u64 each
  int hub_words;
  // forward adjacency (micro tables, X rows), or NULL: vertex v's neighbours
  // after v in the peel order at fadj[rp[v] .. rp[v] + fdeg[v]), in id order
  const int* fadj;
  const int* fdeg;
};

// Clears words u64 at p.
hipError_t mce_launch_zero(u64* p, size_t words, hipStream_t s);
// Input checks.
hipError_t mce_launch_validate(int n, long long nnz, const int* rp, const int* ci, MceCtl* ctl, int blocks,
                               hipStream_t s);
// tcol (tcap 16-bit entries) and tcrow (mce_peel_tail_rows() ints): the residual
// graph that block 0 of a grid peel finishes on once few vertices remain; tcap 0
// keeps the grid to the end. split (grid peel with a tail): the tail runs as a
// second, one-block launch, and `handed` (if not NULL) is recorded between the
// two; ctl->tail_go then says whether the grid handed anything over, and snap
// (n bytes, cleared by the caller) holds 1 for every vertex still present then.
hipError_t mce_launch_peel(int n, const int* rp, const int* ci, int* deg, int* rnd, int* core, int* alive0,
                           int* alive1, int* front0, int* front1, int* bfront0, int* bfront1, MceCtl* ctl,
                           u64 budget, unsigned short* tcol, long long tcap, int* tcrow, int blocks, int split,
                           unsigned char* snap, hipEvent_t handed, hipStream_t s);
int mce_peel_tail_rows();
int mce_peel_max_blocks(int num_cu);
// roots == NULL: the roots are 0 .. nroots-1. fwd == NULL: first-level roots,
// tallied per sub-class; else the later-neighbour counts go to fwd (u64) and
// the second-level roots are tallied by mce_launch_l2_roots.
// Forward adjacency: fadj[rp[v] .. rp[v] + fdeg[v]) = the neighbours of v after
// v in the peel order, in id order. flong: n ints of scratch (the long rows' list).
// tctl (a split peel's control block): nothing is done unless its grid handed
// a tail over (rnd is then the hand-over order's ranks, mce_launch_search_rank).
hipError_t mce_launch_forward_adj(int n, const int* rp, const int* ci, const int* rnd, int* fadj, int* fdeg,
                                  int* flong, MceCtl* ctl, int blocks, hipStream_t s, const MceCtl* tctl = nullptr);
// A split peel's hand-over order as ranks compared like rounds (srank, n ints):
// the round of a vertex gone before the tail; r0 + the degree handed over for a
// vertex still in it (snap 1). Nothing if the grid handed no tail over.
hipError_t mce_launch_search_rank(int n, const int* rnd, const int* deg, const unsigned char* snap,
                                  const MceCtl* tctl, int* srank, int blocks, hipStream_t s);
// fdeg: the forward adjacency's row lengths, when every vertex is a root of a
// first-level run (roots == NULL, fwd == NULL): |P| is read from it.
hipError_t mce_launch_orient(int n, const int* rp, const int* ci, const int* rnd, const int* roots, int nroots,
                             int* pcount, int* xcount, MceCtl* ctl, u64* fwd, const int* fdeg, int blocks,
                             hipStream_t s);
// The roots of a split peel's hand-over order (fdeg: its forward degrees), all
// of them: |P| and |X| into pcount / xcount (n each), the sub-class tallies,
// largest |P| / |X|, isolated vertices into ctl (a control block of its own),
// with tctl's tail_go, tail_r0, max_degree and the level reached (as
// `degeneracy`) copied there.
hipError_t mce_launch_orient_handover(int n, const int* rp, const int* fdeg, const MceCtl* tctl, int* pcount,
                                      int* xcount, MceCtl* ctl, int blocks, hipStream_t s);
// Second-level roots (Algorithm 4) of the vertex roots: COO sources (src, nnz),
// the forward edges as CSR positions (eroots, at most nnz; their number goes to
// ctl->l2_roots), and per root |P| and |X| (pcount, xcount) and the tallies.
// fwd holds the vertex roots' later-neighbour counts; fwd_tmp mce_scan_temp_words(nroots).
// maxhubs > 0: hub_id (n) and bm (maxhubs x ceil(n / 64) u64) hold the
// adjacency bitmaps that mce_launch_hubs built, for the row tests.
// Adjacency bitmaps of up to maxhubs vertices of degree >= HUB_MIN_DEG: hub_id
// (n ints, -1: none), hub_v (maxhubs), bm (maxhubs x ceil(n / 64) u64); the
// number of candidates goes to ctl->nhubs.
hipError_t mce_launch_hubs(int n, const int* rp, const int* ci, int* hub_id, int* hub_v, u64* bm, int maxhubs,
                           MceCtl* ctl, int blocks, hipStream_t s);
hipError_t mce_launch_l2_roots(int n, long long nnz, const int* rp, const int* ci, const int* rnd,
                               const int* roots, int nroots, u64* fwd, u64* fwd_tmp, int* src, int* eroots,
                               int* pcount, int* xcount, int* hub_id, int* hub_v, u64* bm, int maxhubs,
                               MceCtl* ctl, int blocks, hipStream_t s);
// Groups the roots by sub-class into `lists` and writes each one's table size
// (u64 words) at the same position of `words`.
hipError_t mce_launch_bucket(const int* roots, int nroots, const int* pcount, const int* xcount, int mode,
                             int micro, SubOffsets off, int* lists, u64* words, MceCtl* ctl, int blocks,
                             hipStream_t s);
// In-place exclusive prefix sum of n u64 values; tsum holds mce_scan_temp_words(n) words.
int mce_scan_temp_words(int n);
hipError_t mce_launch_scan(u64* a, int n, u64* tsum, hipStream_t s);

// One wavefront per root (prm.parts == 0), or the split build: a head kernel for
// the ids and hash terms, then a rows kernel over nroots * parts blocks.
hipError_t mce_launch_build(const BuildParams& prm, int blocks, hipStream_t s);

// nroots, num_cu: the launch's roots and the device's CUs (a heavy sub-class of
// few roots stages its tables in LDS when they fit)
SearchLayout mce_search_layout(int sub, int mode, int pcap, int xcap, int rcap, int nroots, int num_cu,
                               bool force_hbm, bool counters);
// Resident wavefronts of a search layout over the whole chip (0 on error).
int mce_search_max_workers(const SearchLayout& L, int num_cu);
hipError_t mce_launch_search(const SearchLayout& L, const SearchParams& prm, hipStream_t s);
// Clears the worker list for nworkers waves and their counter rows (nworkers * MCE_NSTAT u64).
hipError_t mce_launch_wl_init(MceWl* wl, int nworkers, u64* stats, hipStream_t s);

int mce_micro_mail_words();
int mce_micro_max_workers(bool counters, int num_cu);
hipError_t mce_launch_micro(bool counters, const MicroParams& prm, hipStream_t s);
