// Device-side building blocks shared by the engine's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned long long u64;
typedef unsigned int u32;

#define MCE_WAVE 64
#define MCE_GOLDEN 0x9E3779B97F4A7C15ULL

// engine error bits, above the MCE_GRAPH_* input classes (bits 0..4)
#define MCE_E_TIMEOUT (1u << 16)   // a bounded wait or the search ran past its deadline
#define MCE_E_LIMIT (1u << 17)     // a root's P does not fit the launch's bitset width
#define MCE_E_PROTO (1u << 18)     // worker-list bookkeeping went wrong
#define MCE_E_ROOTS (1u << 19)     // a root id outside [0, n)
#define MCE_E_HEAP (1u << 20)      // the induced-subgraph heap was too small
#define MCE_E_MSTACK (1u << 21)    // a micro frame stack overflowed (the engine runs again with larger ones)
// a search kernel that finds any of these set searches nothing more
#define MCE_E_STOP (MCE_E_HEAP | MCE_E_LIMIT | MCE_E_TIMEOUT | MCE_E_MSTACK)

// Bitset-width classes: widths 1, 2, 4, 8, 16, 32 words of 64 bits (P up to 2048).
#define MCE_NCLASS 6
#define MCE_MAX_P 2048
#define MCE_MAX_WORKERS 8192
// Sub-classes: a width class split by whether a root's induced subgraph (rows
// and X_X array) is staged in LDS ("light") or read from HBM ("heavy"), plus the
// micro sub-class: |P| <= 64 and |X| <= 64, searched one frame per lane.
#define MCE_SUB_MICRO (2 * MCE_NCLASS)
#define MCE_NSUB (2 * MCE_NCLASS + 1)
#define MCE_MICRO_MAX 64
#ifndef MCE_LIGHT_BYTES
#define MCE_LIGHT_BYTES 4096   // largest staged rows + X_X array of a "light" root
#endif
// classification variants tallied by the orientation: mode | (micro off << 1)
#define MCE_NVAR 4
// pivot keys pack (count << 20 | ~local index): local indices stay below 2^20
#define MCE_MAX_LOCAL ((1 << 20) - 1)

// Induced-subgraph modes (section 3.4 of the pages): partial (P x P rows, P-X
// edges looked up in the CSR) or full (P x (P u X) rows).
#define MCE_MODE_IP 0
#define MCE_MODE_IPX 1

__host__ __device__ inline int mce_class_of(int p) {   // smallest class whose 64*W >= p
  int c = 0;
  while (c < MCE_NCLASS - 1 && (64 << c) < p) c++;
  return c;
}

// Rows of a root's induced subgraph: P rows only (IP) or P and X rows (IPX).
__host__ __device__ inline long long mce_table_rows(int p, int x, int mode) {
  return mode == MCE_MODE_IPX ? (long long)p + x : (long long)p;
}

// Words (u64) of a root's table in the heap:
//   [0] p | x << 32    [1] root id | |R| << 32    [2] hash terms of R summed
//   [3 .. 3 + rows*W)  bit rows over the root's P (local index order = id order)
//   then p hash terms of the P members, then p + x int32 ids (P ids, X ids).
__host__ __device__ inline unsigned long long mce_table_words(int p, int x, int W, int mode) {
  return 3ull + (unsigned long long)mce_table_rows(p, x, mode) * (unsigned long long)W + (unsigned long long)p +
         ((unsigned long long)p + (unsigned long long)x + 1ull) / 2ull;
}

// LDS bytes that staging a root's rows and X_X array takes.
__host__ __device__ inline unsigned long long mce_stage_bytes(int p, int x, int W, int mode) {
  return (unsigned long long)mce_table_rows(p, x, mode) * (unsigned long long)W * 8ull +
         (unsigned long long)x * 4ull;
}

__host__ __device__ inline bool mce_is_micro(int p, int x) { return p <= MCE_MICRO_MAX && x <= MCE_MICRO_MAX; }

// Micro table: the full table's header and P u X rows, then for each P member
// the bitset of the X members adjacent to it, the P hash terms and the ids.
__host__ __device__ inline unsigned long long mce_micro_table_words(int p, int x) {
  return 3ull + (unsigned long long)(p + x) + 2ull * (unsigned long long)p + ((unsigned long long)(p + x) + 1ull) / 2ull;
}

__host__ __device__ inline int mce_sub_of(int p, int x, int mode, bool micro) {
  if (micro && mce_is_micro(p, x)) return MCE_SUB_MICRO;
  const int c = mce_class_of(p);
  return 2 * c + (mce_stage_bytes(p, x, 1 << c, mode) > MCE_LIGHT_BYTES ? 1 : 0);
}

__host__ __device__ inline unsigned long long mce_sub_table_words(int p, int x, int sub, int mode) {
  if (sub == MCE_SUB_MICRO) return mce_micro_table_words(p, x);
  return mce_table_words(p, x, 1 << (sub >> 1), mode);
}

#define MCE_BAR_GROUPS 16   // grid barrier: block groups with a counter each
#define MCE_BAR_STRIDE 32   // u32 words from one barrier counter to the next (a 128-byte line)

// Control block: one per run, zeroed by the host before the first kernel.
struct MceCtl {
  u32 status;            // MCE_GRAPH_* | MCE_E_*
  int max_degree;
  int degeneracy;
  int rounds;
  int max_p;
  int max_x;
  int min_deg[2];        // peel: smallest degree in each remaining list (by list parity)
  u64 isolated;          // roots of degree 0
  u64 isolated_hash;     // sum of their clique hashes
  u64 pairs;             // second-level roots {r, w} with P and X empty: maximal cliques of size 2
  u64 pairs_hash;        // sum of their clique hashes
  int l2_roots;          // second-level roots (forward edges of the vertex roots)
  int nhubs;             // vertices of degree >= HUB_MIN_DEG seen (the first ones get an adjacency bitmap)
  int nlong;             // forward adjacency: rows too long for one wavefront, listed for the second pass
  // per classification variant (subgraph mode, micro sub-class on/off) and
  // sub-class: roots, largest |P|, largest |X|, largest row count, heap words
  int sub_count[MCE_NVAR][MCE_NSUB];
  int sub_maxp[MCE_NVAR][MCE_NSUB];
  int sub_maxx[MCE_NVAR][MCE_NSUB];
  int sub_maxr[MCE_NVAR][MCE_NSUB];   // largest row count of a table
  u64 sub_words[MCE_NVAR][MCE_NSUB];
  int sub_cursor[MCE_NSUB];
  int asize[2];          // peel: alive-list sizes (ping-pong)
  int fsize[3];          // peel: frontier sizes, one slot per step (rotating: read, filled, being reset)
  int bsize[3];          // peel: big-vertex frontier sizes (same rotation)
  int bedge[3];          // peel: the big vertices' CSR row lengths summed (same rotation)
  int asum[2];           // peel: each remaining list's CSR row lengths summed (by list parity)
  int tmax[2];           // peel: each remaining list's largest degree (by list parity; short lists only)
  u64 tsum[2];           // peel: the compacted residual graph's size in 16-bit entries (same)
  int tlong;             // peel compaction: remaining vertices whose rows are written in spans
  int tpad;
  u32 vpad;
  u32 vdone;             // validation: blocks of the entry pass that finished
  u64 vdown, vup;        // validation: edges from the larger (degree, id) end, and from the smaller
  u32 seg_gen;           // peel: segments of tiny rounds that block 0 has handed back
  u32 seg_arrive;        // peel: blocks that started waiting for a segment (summed over segments)
  int seg_state[12];     // peel: the state block 0 hands back (result, list, frontier, level, round, slot, sums)
  u64 t_run;             // wall-clock tick at the start of the peel: the run's time limit counts from it
  u64 peel_ticks[4];     // block 0 of the peel: barrier waits, level passes, round work, total
  // split peel (the grid stops where block 0 would go on alone on the compacted
  // residual graph, and k_peel_tail goes on from here in a launch of its own)
  int tail_go;           // 1: the grid handed over, with the state below
  int tail_r0;           // the tail's first round: every vertex with a smaller round has left
  int tail_st[4];        // level, round, vertices left, which remaining list
  u64 tail_ticks[3];     // block 0's barrier, level and round ticks up to the hand-over
  u32 taken[2 * MCE_NCLASS + 2];   // per search launch: subtrees handed out (see record_taken); the
                                   // last one is the split peel's early launch's
  // grid barrier of the peel, one 128-byte line each: [0] groups complete,
  // [1] barriers released, [2 + g] arrivals of block group g (all counts since
  // the launch began)
  alignas(128) u32 bar[(2 + MCE_BAR_GROUPS) * MCE_BAR_STRIDE];
};

// Worker-list state of one search launch (section 3.3 of the pages). Each
// wavefront owns one 128-byte line: word 0 is its wake flag, word 16 its
// request word. A wave that runs out of work closes its request word, gives up
// its share of n_active and asks busy waves for branches: it picks a wave at
// random and, if that wave's request word is open (0), writes its own id + 1
// there with a compare-and-swap, then sleeps on its wake flag. A busy wave
// reads only its own request word (once per search-tree node) and answers with
// a branch (MCE_FLAG_TASK, after counting the receiver active) or with
// MCE_FLAG_RETRY. Every hot word is private to one wave, so no atomic is
// contended by thousands of waves. A bitmap of the open request words lets an
// idle wave pick a busy wave in one read instead of probing idle ones; it is
// only a hint (the compare-and-swap on the request word decides).
//
// Termination does not assume that every wavefront of the grid is resident: a
// wavefront counts in n_active only while it holds a task or is about to take a
// first-level subtree, and request words start closed. The wavefront whose
// release brings n_active to zero writes MCE_FLAG_EXIT into every wake flag; a
// wave that starts later finds the roots gone and leaves the same way.
#define MCE_LINE_WORDS 32     // u32 words per 128-byte line
#define MCE_REQ_WORD 16       // first request slot inside a wave's line
#define MCE_REQ_SLOTS 4       // request slots per wave (the micro kernel answers up to four per step)
#define MCE_FLAG_TASK 1u
#define MCE_FLAG_EXIT 2u
#define MCE_FLAG_RETRY 3u
#define MCE_REQ_CLOSED 0xFFFFFFFFu
struct MceWl {
  u32 root_ctr;          // next first-level subtree to hand out (phase 1)
  u32 pad0[MCE_LINE_WORDS - 1];
  int n_active;          // wavefronts holding (or about to take) a task
  u32 pad1[MCE_LINE_WORDS - 1];
  u32 done;              // set on abort (time limit or protocol error)
  u32 pad2[MCE_LINE_WORDS - 1];
  // bit w of word w / 64 (one word per 128-byte line): wave w's request word is
  // open, a hint for askers
  u64 open_mask[MCE_MAX_WORKERS / 64 * 16];
  u32 line[MCE_MAX_WORKERS * MCE_LINE_WORDS];   // wave w: flag at [w*32], request at [w*32 + 16]
};

// ---------------------------------------------------------------- hashing
__device__ __forceinline__ u64 mce_mix64(u64 z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}
__device__ __forceinline__ u64 mce_vertex_term(int v) { return mce_mix64((u64)(long long)v + MCE_GOLDEN); }
__device__ __forceinline__ u64 mce_clique_term(u64 sum, int k) { return mce_mix64(sum + (u64)k * MCE_GOLDEN); }

// ---------------------------------------------------------------- lanes
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
__device__ __forceinline__ u64 ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
__device__ __forceinline__ int mbcnt(u64 m) {   // set bits of m below this lane
  return __builtin_amdgcn_mbcnt_hi((u32)(m >> 32), __builtin_amdgcn_mbcnt_lo((u32)m, 0u));
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ u32 uni(u32 x) { return (u32)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ u64 uni(u64 x) {
  u32 lo = (u32)__builtin_amdgcn_readfirstlane((int)(u32)x);
  u32 hi = (u32)__builtin_amdgcn_readfirstlane((int)(u32)(x >> 32));
  return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ u64 read_lane(u64 x, int l) {
  u32 lo = (u32)__builtin_amdgcn_readlane((int)(u32)x, l);
  u32 hi = (u32)__builtin_amdgcn_readlane((int)(u32)(x >> 32), l);
  return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ int read_lane(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// Whole-wave reductions with DPP row operations, result in every lane.
// Must be called with all 64 lanes active.
template <int CTRL, int ROWS>
__device__ __forceinline__ u32 dpp_u32(u32 v) {
  return (u32)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
#define MCE_DPP_REDUCE(NAME, OP)                                   \
  __device__ __forceinline__ u32 NAME(u32 x) {                     \
    x = OP(x, dpp_u32<0xB1, 0xF>(x));   /* quad_perm 1,0,3,2 */    \
    x = OP(x, dpp_u32<0x4E, 0xF>(x));   /* quad_perm 2,3,0,1 */    \
    x = OP(x, dpp_u32<0x141, 0xF>(x));  /* row_half_mirror  */     \
    x = OP(x, dpp_u32<0x140, 0xF>(x));  /* row_mirror       */     \
    x = OP(x, dpp_u32<0x142, 0xA>(x));  /* row_bcast15 -> rows 1,3 */ \
    x = OP(x, dpp_u32<0x143, 0xC>(x));  /* row_bcast31 -> rows 2,3 */ \
    return (u32)__builtin_amdgcn_readlane((int)x, 63);            \
  }
__device__ __forceinline__ u32 op_max(u32 a, u32 b) { return a > b ? a : b; }
__device__ __forceinline__ u32 op_add(u32 a, u32 b) { return a + b; }
__device__ __forceinline__ u32 op_or(u32 a, u32 b) { return a | b; }
MCE_DPP_REDUCE(wave_max_u32, op_max)
MCE_DPP_REDUCE(wave_sum_u32, op_add)
MCE_DPP_REDUCE(wave_or_u32, op_or)
__device__ __forceinline__ u64 wave_sum_u64(u64 x) {   // via 16/16/32-bit pieces, carries kept
  u32 lo = (u32)x, hi = (u32)(x >> 32);
  u32 l0 = wave_sum_u32(lo & 0xFFFFu);
  u32 l1 = wave_sum_u32(lo >> 16);
  u32 h = wave_sum_u32(hi);
  return ((u64)h << 32) + ((u64)l1 << 16) + (u64)l0;
}
__device__ __forceinline__ int wave_min_i32_nonneg(int x) {   // x >= 0 in every lane
  return (int)(0x7FFFFFFFu - wave_max_u32(0x7FFFFFFFu - (u32)x));
}

// ---------------------------------------------------------------- scoped atomics
__device__ __forceinline__ u32 ld_relaxed(const u32* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_relaxed(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 ld_acquire(const u32* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(u32* p, u32 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(u32* p, u32 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_relaxed64(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed64(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed_i(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed. Agent-scope
// relaxed atomic stores (sc1) are performed at the device coherence point, so
// once this wait returns they are visible to agent-scope atomic loads of any
// wave. Publishing data as "atomic stores, wait, flag store" replaces an
// agent-scope release fence, whose L2 write-back serialises across the chip
// when thousands of waves issue it. The signal fences keep the compiler from
// moving memory operations across the wait.
__device__ __forceinline__ void wait_stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_acq_rel_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent"); }

// ---------------------------------------------------------------- CSR lookups
// Is key in the sorted range ci[lo, hi)?
__device__ __forceinline__ bool csr_range_has(const int* __restrict__ ci, int lo, int hi, int key) {
  int len = hi - lo;
  while (len > 0) {
    int half = len >> 1;
    int mid = lo + half;
    if (ci[mid] < key) {
      lo = mid + 1;
      len -= half + 1;
    } else {
      len = half;
    }
  }
  return lo < hi && ci[lo] == key;
}

// Are x and y adjacent? Searches the shorter of the two rows.
__device__ __forceinline__ bool csr_adjacent(const int* __restrict__ rp, const int* __restrict__ ci,
                                             int x, int y) {
  int xa = rp[x], xb = rp[x + 1];
  int ya = rp[y], yb = rp[y + 1];
  if (xb - xa <= yb - ya) return csr_range_has(ci, xa, xb, y);
  return csr_range_has(ci, ya, yb, x);
}

// "u comes after v" in the degeneracy order (round, id).
__device__ __forceinline__ bool order_after(int ru, int u, int rv, int v) {
  return ru > rv || (ru == rv && u > v);
}

__device__ __forceinline__ bool past_deadline(u64 deadline) { return wall_clock64() > deadline; }
