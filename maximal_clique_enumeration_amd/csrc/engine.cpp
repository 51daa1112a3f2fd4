// Host side of the engine: the C ABI declared in include/mce.h.
//
// One mce_run queues, on the caller's stream: CSR validation, the k-core peel
// (degeneracy order, "Parallelizing Maximal Clique Enumeration on GPUs" section
// 2.4), the per-root P/X split, then one persistent search launch per bitset
// width class (sections 3.1-3.5), and reads back count, histogram and hash.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/mce.h"
#include "mce_internal.h"

namespace {

struct DevBuf {
  void* p = nullptr;
  size_t bytes = 0;
};

struct HostPinned {
  void* p = nullptr;
  size_t bytes = 0;
};

// Every device buffer of a run. An engine has two sets: its own, grown with
// hipMalloc and kept until mce_destroy, and one carved out of the device's
// static scratch array by mce_run_static.
struct Bufs {
  DevBuf ctl, deg, rnd, core, alive0, alive1, front0, front1, bfront0, bfront1, pcount, xcount, lists, taboff, scan,
      heap, wl, slots, stats, mstack, mail;
  DevBuf src, fwd, fwdtmp, eroots, pcount2, xcount2;   // second-level subtrees
  DevBuf hub_id, hub_v, hub_bm;                       // their hub adjacency bitmaps
  DevBuf fadj, fdeg, flong;                           // forward adjacency (table builds)
  DevBuf tcol, tcrow;                                 // the peel's compacted residual graph
  // the early launch of a split peel (the roots that left before the tail)
  DevBuf ctl1, snap, srank, fadj1, fdeg1, flong1, pcount1, xcount1;
};

constexpr size_t kHistWords = MCE_MAX_P + 3;   // global histogram entries (sizes up to 2 + MCE_MAX_P)
// control block, then the result words (hash, histogram): one clear, one read-back
constexpr size_t kIoBytes = sizeof(MceCtl) + (1 + kHistWords) * sizeof(u64);
static_assert(sizeof(MceCtl) % sizeof(u64) == 0, "results follow the control block");
constexpr int kOccSlots = 64;   // cached occupancy answers per engine

// Bump allocation over the static scratch (mce_run_static): buffers are laid
// out afresh by every run, 256-byte aligned.
struct Arena {
  char* base = nullptr;   // nullptr: the engine's own hipMalloc'd buffers
  size_t cap = 0, used = 0, need = 0;
  bool short_of_space = false;
};

}  // namespace

struct mce_engine {
  mce_config cfg;
  int device = 0;
  int num_cu = 0;
  double tick_hz = 100e6;
  int peel_blocks_max = 1;
  char err[512] = {0};

  Bufs own;           // grown with hipMalloc, freed by mce_destroy
  Bufs carved;        // the static scratch, laid out by the last mce_run_static
  Bufs* last = &own;  // the set the last run used (mce_ordering, mce_stats)
  HostPinned host;    // staging for device -> host copies (mce_run, mce_run_roots)
  alignas(64) unsigned char host_io[kIoBytes];   // the same for mce_run_static (pageable)
  hipEvent_t ev[4 + 4 * MCE_NSUB] = {};
  bool have_events = false;
  // the overlapped search launches: streams forked from the caller's stream
  // (fork_ev) and joined back to it (join_ev)
  hipStream_t side[MCE_SIDE_STREAMS] = {};
  hipEvent_t fork_ev = nullptr;
  hipEvent_t join_ev[MCE_SIDE_STREAMS] = {};
  // a split peel's hand-over order is set up on side stream 0 from the grid's
  // hand-over (handed_ev); its control block is read back through host1
  hipEvent_t handed_ev = nullptr;
  HostPinned host1;

  // last run
  bool have_result = false;
  bool complete = false;      // false: the search stopped at the time limit; the results are partial
  bool have_order = false;
  int32_t last_n = 0;
  uint64_t count = 0, hash = 0;
  uint64_t hist[kHistWords] = {};
  int32_t hist_len = 0;
  mce_graph_facts info{};
  mce_run_stats stats_out{};
  std::vector<mce_worker_record> trace;   // filled on demand by mce_stats / mce_worker_trace

  // per-wave counters of the last run stay on the device until mce_stats or
  // mce_worker_trace asks for them (they are diagnostics, not results)
  struct LaunchInfo {
    int sub, nw, roots;
  };
  LaunchInfo last_plan[MCE_NSUB] = {};
  // where the last run's induced-subgraph tables sit (mce_root_table): valid
  // after a complete first-level run with overlapped launches, each sub-class
  // in its own heap region
  struct TableMap {
    bool valid = false;
    int mode = 0;
    int total = 0;                      // root-list entries
    int off[MCE_NSUB] = {}, count[MCE_NSUB] = {};
    size_t heap_base[MCE_NSUB] = {};    // u64 words
  } tabs;
  int n_last_plan = 0;
  int last_stat_rows = 0;
  bool stats_pending = false;
  bool last_timing = false;
  bool last_stimes = false;   // the search launches carry events (MCE_FLAG_SEARCH_TIMES or _PHASE_TIMES)
  // resident-wave counts per kernel variant (occupancy queries cost ~0.1 ms each)
  struct Occ {
    int a;
    long long b;
    int v;
  };
  Occ occ[kOccSlots] = {};
  int n_occ = 0;
  int micro_stack = 4096;   // micro frame stack of mce_run / mce_run_roots, frames per wave (grows)
};

namespace {

mce_status fail(mce_engine* e, mce_status s, const char* fmt, ...) {
  if (e) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(e->err, sizeof(e->err), fmt, ap);
    va_end(ap);
  }
  return s;
}

mce_status hip_fail(mce_engine* e, hipError_t h, const char* what) {
  return fail(e, h == hipErrorOutOfMemory ? MCE_ERR_NOMEM : MCE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(h));
}

hipError_t ensure(DevBuf& b, size_t bytes) {
  if (bytes == 0) bytes = 1;
  if (b.bytes >= bytes) return hipSuccess;
  if (b.p) (void)hipFree(b.p);
  b.p = nullptr;
  b.bytes = 0;
  hipError_t h = hipMalloc(&b.p, bytes);
  if (h == hipSuccess) b.bytes = bytes;
  return h;
}

// A buffer of the run: the engine's own (grown with hipMalloc) or, with an
// arena, the next piece of the static scratch (no allocation call).
hipError_t take(Arena& a, DevBuf& b, size_t bytes) {
  if (!a.base) return ensure(b, bytes);
  if (bytes == 0) bytes = 1;
  const size_t off = (a.used + 255) & ~(size_t)255;
  if (off + bytes > a.cap) {
    a.short_of_space = true;
    a.need = std::max(a.need, off + bytes);
    return hipErrorOutOfMemory;
  }
  b.p = a.base + off;
  b.bytes = bytes;
  a.used = off + bytes;
  return hipSuccess;
}

// An allocation failure: with the static scratch it means the run does not fit
// (MCE_ERR_LIMIT, with the bytes it needed at least); else the device's.
mce_status alloc_fail(mce_engine* e, const Arena& a, hipError_t h, const char* what) {
  if (a.base && a.short_of_space)
    return fail(e, MCE_ERR_LIMIT, "%s: the static scratch holds %zu bytes; this run needs more than %zu", what,
                a.cap, a.need);
  return hip_fail(e, h, what);
}

hipError_t ensure_host(HostPinned& b, size_t bytes) {
  if (b.bytes >= bytes) return hipSuccess;
  if (b.p) (void)hipHostFree(b.p);
  b.p = nullptr;
  b.bytes = 0;
  hipError_t h = hipHostMalloc(&b.p, bytes, hipHostMallocDefault);
  if (h == hipSuccess) b.bytes = bytes;
  return h;
}

void release(DevBuf& b) {
  if (b.p) (void)hipFree(b.p);
  b.p = nullptr;
  b.bytes = 0;
}

template <class T>
T* dp(DevBuf& b) {
  return static_cast<T*>(b.p);
}

double ms_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

// Occupancy answer for a kernel variant, cached per engine (fixed table: the
// run path allocates nothing on the host either).
template <class F>
int occupancy(mce_engine* e, int a, long long b, F query) {
  for (int i = 0; i < e->n_occ; i++)
    if (e->occ[i].a == a && e->occ[i].b == b) return e->occ[i].v;
  const int v = query();
  if (e->n_occ < kOccSlots) e->occ[e->n_occ++] = {a, b, v};
  return v;
}

constexpr int kMaxHubs = 1024;                 // second-level orientation: hub adjacency bitmaps, at most
constexpr size_t kHubBytes = 256ull << 20;     // this many, in at most this many bytes
constexpr int kMicroStack = 4096;              // frames per wavefront stack of the micro search, to start with
constexpr int kMicroStackMax = 1 << 20;        // ... grown 4x after an overflow, up to this many
constexpr int kMicroStackMinStatic = 256;      // the smallest stack mce_run_static gives a micro wave
// The peel finishes in block 0 on the residual graph compacted to 16-bit local
// ids once at most this many entries remain (96 MB): one compute unit reads
// them all, and past this it would take longer than the grid's rounds.
#ifndef MCE_PEEL_TAIL_ENTRIES
#define MCE_PEEL_TAIL_ENTRIES (48ll << 20)
#endif
#ifndef MCE_MICRO_COOP_ROOTS_PER_WAVE
#define MCE_MICRO_COOP_ROOTS_PER_WAVE 4
#endif
#ifndef MCE_BUILD_BLOCKS_PER_CU
#define MCE_BUILD_BLOCKS_PER_CU 32   // micro build: one-wave blocks per CU; the split build's kernels a quarter of it
#endif
#ifndef MCE_MICRO_WAVES_PER_CU
#define MCE_MICRO_WAVES_PER_CU 8
#endif
#ifndef MCE_MICRO_WAVES_PER_CU_BESIDE
#define MCE_MICRO_WAVES_PER_CU_BESIDE 3
#endif
// Micro launches keep at most 8 wavefronts per CU alone (more add start-up
// spread and little throughput), 3 beside other launches, which then get the
// compute units: the 500k Chung-Lu graph at 8 / 5 / 4 / 3 / 2 waves per CU
// beside the others, 17.14 / 16.90 / 16.88 / 16.85 / 17.70 ms a step (3 against
// 4 in three more comparisons: 0.07-0.08 ms faster; the 4M-vertex uniform
// sample 62.61 -> 62.37 ms); in series, 23.65 ms at 8 and 25.57 ms at 4.
// micro launches with this many roots per wave share pivot scans
constexpr int kMicroCoopRootsPerWave = MCE_MICRO_COOP_ROOTS_PER_WAVE;
#ifndef MCE_W1_WAVES_PER_CU
#define MCE_W1_WAVES_PER_CU 8
#endif
// Width-1 launches keep at most this many wavefronts per CU. Their waves are
// fast and soon idle, and every idle wave asks the busy ones for branches, so
// more of them cost the waves that hold the work more than they add (the 500k
// Chung-Lu graph's 143 and 20,491 width-1 roots: 2.3 and 2.2 ms with 28 waves
// per CU, 1.1 and 0.9 ms with 8).
constexpr int kW1WavesPerCu = MCE_W1_WAVES_PER_CU;
#ifndef MCE_W1_WAVES_PER_CU_BESIDE
#define MCE_W1_WAVES_PER_CU_BESIDE 4
#endif
// ... and this many beside other launches, where the waves they leave free go
// to the width-2 launch that sets the step's length (the 500k Chung-Lu graph:
// 17.24 / 17.11 / 17.11 / 17.08 ms a step at 8 / 6 / 5 / 4 waves per CU; alone,
// 4 waves per CU made the width-1 launches slower, 23.56 -> 23.8 ms a step with
// the launches in series).
constexpr int kW1WavesPerCuBeside = MCE_W1_WAVES_PER_CU_BESIDE;
// Tables other than micro ones are built by the split build: a root's rows are
// dealt over several blocks, about this many (root, part) blocks per CU.
#ifndef MCE_SPLIT_BLOCKS_PER_CU
#define MCE_SPLIT_BLOCKS_PER_CU 16
#endif
constexpr int kSplitBlocksPerCu = MCE_SPLIT_BLOCKS_PER_CU;
#ifndef MCE_WIDE_WAVES_PER_CU
#define MCE_WIDE_WAVES_PER_CU 14
#endif
// Wider launches beside other launches keep at most this many wavefronts per
// CU. A search launch is persistent: its waves hold their compute units until
// the launch's work is done, so a launch queued on another side stream that
// finds no room waits for it. The 500k Chung-Lu graph's width-2 launch filled
// 17 waves per CU (its LDS limit) and the width-1 chains ran after it (19.7 ms a
// step); capped at 10 / 12 / 13 / 14 / 15 / 16 waves: 19.2 / 18.6 / 18.4 /
// 18.2 / 18.7 / 19.5 ms.
constexpr int kWideWavesPerCu = MCE_WIDE_WAVES_PER_CU;




// ------------------------------------------------------------------ static scratch
// The device memory of mce_run_static: one array per device, holding every
// buffer of a run (partial results, counters, queues, stacks, tables), kept
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress, once
// per device (mce_create, with that device current), and only that address is
// used (kernel arguments, clears).
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;      // guards g_scratch_ptr
std::mutex g_static_run_mu;   // held by every mce_run_static call

}  // namespace

static __device__ __align__(256) unsigned char scratch[MCE_STATIC_SCRATCH_BYTES];

namespace {

hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t h = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (h != hipSuccess) return h;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// One run. `arena` empty: the engine's own buffers (grown with hipMalloc);
// else every buffer is carved from the static scratch and nothing is allocated.
// One attempt of a run. *grow: the micro kernel's frame stacks overflowed, and
// the run should be made again with larger ones.
mce_status run_once(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                    const int32_t* roots, int32_t nroots, bool subset, void* stream, Arena& arena, bool* grow) {
  const auto t0 = std::chrono::steady_clock::now();
  if (!e) return MCE_ERR_ARG;
  const bool stat = arena.base != nullptr;
  Bufs& B = stat ? e->carved : e->own;
  e->last = &B;
  e->err[0] = 0;
  e->have_result = false;
  e->complete = false;
  e->have_order = false;
  e->tabs.valid = false;
  if (n < 0 || nnz < 0) return fail(e, MCE_ERR_ARG, "n and nnz must be >= 0");
  if (nnz >= 0x7FFFFFFFLL) return fail(e, MCE_ERR_ARG, "nnz must be < 2^31");
  if (n > 0 && !row_ptr) return fail(e, MCE_ERR_ARG, "row_ptr is NULL");
  if (nnz > 0 && !col_idx) return fail(e, MCE_ERR_ARG, "col_idx is NULL");
  if (subset && (nroots < 0 || (nroots > 0 && !roots))) return fail(e, MCE_ERR_ARG, "bad roots");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t h = hipSetDevice(e->device);
  if (h != hipSuccess) return hip_fail(e, h, "hipSetDevice");

  e->stats_pending = false;
  e->info = mce_graph_facts{};
  e->info.n = n;
  e->info.nnz = nnz;
  std::memset(&e->stats_out, 0, sizeof(e->stats_out));
  e->stats_out.struct_size = sizeof(mce_run_stats);
  e->stats_out.tick_hz = e->tick_hz;
  e->hist_len = 0;
  e->count = e->hash = 0;
  e->last_n = n;
  const int cnt = subset ? nroots : n;
  e->info.roots = cnt;
  if (n == 0) {
    if (subset && nroots > 0) return fail(e, MCE_ERR_ARG, "roots given for an empty graph");
    e->have_result = true;
    e->complete = true;
    e->info.complete = 1;
    e->stats_out.ms_total = ms_since(t0);
    return MCE_OK;
  }
  const bool timing = (e->cfg.flags & MCE_FLAG_PHASE_TIMES) && e->have_events;
  // events around the search launches only (every recorded event costs the stream a few us)
  const bool stimes = (timing || (e->cfg.flags & MCE_FLAG_SEARCH_TIMES)) && e->have_events;
  const bool hbm = (e->cfg.flags & MCE_FLAG_HBM_STAGING) != 0;
  const bool counters_on = (e->cfg.flags & MCE_FLAG_COUNTERS) != 0;
  const u64 budget = (u64)((double)e->cfg.timeout_ms * 1e-3 * e->tick_hz);
  // sub-class launches overlapped on the engine's streams, each with its own
  // heap region, worker list and slots; else one after another, sharing them
  const bool overlap = !stat && (e->cfg.flags & MCE_FLAG_SERIAL) == 0;

  size_t nb = (size_t)n * sizeof(int);
  if ((h = take(arena, B.ctl, kIoBytes)) != hipSuccess || (h = take(arena, B.deg, nb)) != hipSuccess ||
      (h = take(arena, B.rnd, nb)) != hipSuccess || (h = take(arena, B.core, nb)) != hipSuccess ||
      (h = take(arena, B.alive0, nb)) != hipSuccess || (h = take(arena, B.alive1, nb)) != hipSuccess ||
      (h = take(arena, B.front0, nb)) != hipSuccess || (h = take(arena, B.front1, nb)) != hipSuccess ||
      (h = take(arena, B.bfront0, nb)) != hipSuccess || (h = take(arena, B.bfront1, nb)) != hipSuccess ||
      (h = take(arena, B.pcount, (size_t)std::max(cnt, 1) * sizeof(int))) != hipSuccess ||
      (h = take(arena, B.xcount, (size_t)std::max(cnt, 1) * sizeof(int))) != hipSuccess ||
      (h = take(arena, B.wl, sizeof(MceWl) * (overlap ? MCE_NSUB + 1 : 1))) != hipSuccess)
    return alloc_fail(e, arena, h, "allocation");
  if (!stat && (h = ensure_host(e->host, kIoBytes)) != hipSuccess) return hip_fail(e, h, "allocation");
  // second-level subtrees (section 3.2): the roots are the vertex roots' forward edges
  const bool l2 = (e->cfg.flags & MCE_FLAG_L2) != 0;
  e->info.level = l2 ? 2 : 1;
  int maxhubs = 0;
  if (l2) {
    const size_t ne = (size_t)std::max<int64_t>(nnz, 1) * sizeof(int);
    if ((h = take(arena, B.src, ne)) != hipSuccess || (h = take(arena, B.eroots, ne)) != hipSuccess ||
        (h = take(arena, B.pcount2, ne)) != hipSuccess || (h = take(arena, B.xcount2, ne)) != hipSuccess ||
        (h = take(arena, B.fwd, (size_t)std::max(cnt, 1) * sizeof(u64))) != hipSuccess ||
        (h = take(arena, B.fwdtmp, (size_t)mce_scan_temp_words(std::max(cnt, 1)) * sizeof(u64))) != hipSuccess)
      return alloc_fail(e, arena, h, "allocation");
  }
  // hub adjacency bitmaps (second-level runs; first-level builds did not gain
  // from them): n bits each, at most kMaxHubs within kHubBytes. They only change
  // the speed, and the static scratch has no room for them.
  if (l2 && !stat) {
    const size_t hub_bytes = ((size_t)n + 63) / 64 * sizeof(u64);
    maxhubs = (int)std::min<size_t>(kMaxHubs, kHubBytes / std::max<size_t>(hub_bytes, 1));
    if (maxhubs > 0 &&
        ((h = ensure(B.hub_id, (size_t)n * sizeof(int))) != hipSuccess ||
         (h = ensure(B.hub_v, (size_t)maxhubs * sizeof(int))) != hipSuccess ||
         (h = ensure(B.hub_bm, (size_t)maxhubs * hub_bytes)) != hipSuccess))
      return hip_fail(e, h, "allocation");
  }
  // the root lists: one entry per vertex root, or per edge for second-level subtrees
  const size_t lists_cap = l2 ? (size_t)std::max<int64_t>(nnz, 1) : (size_t)std::max(cnt, 1);
  if ((h = take(arena, B.lists, lists_cap * sizeof(int))) != hipSuccess) return alloc_fail(e, arena, h, "allocation");

  MceCtl* ctl = dp<MceCtl>(B.ctl);
  u64* results = reinterpret_cast<u64*>(dp<char>(B.ctl) + sizeof(MceCtl));   // hash, then the histogram
  // cleared by a kernel (the static scratch keeps the last run's contents)
  if ((h = mce_launch_zero(dp<u64>(B.ctl), kIoBytes / sizeof(u64), s)) != hipSuccess) return hip_fail(e, h, "clear");

  const int grid = std::max(1, e->num_cu * 8);
  if (timing) (void)hipEventRecord(e->ev[0], s);
  if (e->cfg.validate) {
    if ((h = mce_launch_validate(n, nnz, row_ptr, col_idx, ctl, grid, s)) != hipSuccess)
      return hip_fail(e, h, "validate launch");
  }
  if (timing) (void)hipEventRecord(e->ev[1], s);
  // the peel: one block for small graphs (no grid barrier traffic), else one
  // block per two CUs (against one per CU: cheaper barriers and still ample
  // waves for a round; configurations 2-4 peel 3-5 % faster)
  int pblocks = n <= 16384 ? 1 : std::min(std::max(1, e->peel_blocks_max / 2), (n + 1023) / 1024);
  // the grid peel's tail: the residual graph compacted for block 0 (not
  // mce_run_static: its scratch is kept for the search; the grid peels to the end)
  long long tcap = 0;
  if (pblocks > 1 && !stat) {
    tcap = std::min<long long>(nnz + nnz / 64 + (1ll << 20), MCE_PEEL_TAIL_ENTRIES);
    if ((h = ensure(B.tcol, (size_t)tcap * sizeof(unsigned short))) != hipSuccess ||
        (h = ensure(B.tcrow, (size_t)mce_peel_tail_rows() * sizeof(int))) != hipSuccess)
      return hip_fail(e, h, "allocation");
  }
  // Split peel: the grid stops where block 0 would finish alone on the
  // compacted residual graph, and the tail runs as a one-block launch of its
  // own. Every vertex gone by then has its final round, and every vertex still
  // in the tail comes after it; the search takes the vertices of the tail
  // among themselves by their degree in the remaining graph (then id) instead
  // of their rounds, so that every subtree is fixed at the hand-over and the
  // whole search runs on the compute units the tail leaves idle (whole-graph
  // first-level runs with overlapped launches). Any vertex order reports each
  // maximal clique once; the degeneracy order is what keeps |P| small, and the
  // tail's vertices are the last ones of it either way.
  const bool micro_on = (e->cfg.flags & MCE_FLAG_NO_MICRO) == 0;
  const bool split = overlap && !l2 && !subset && tcap > 0;
  MceCtl* ctl1 = nullptr;
  if (split) {
    const size_t snap_words = ((size_t)n + 7) / 8;
    if ((h = ensure(B.ctl1, sizeof(MceCtl))) != hipSuccess ||
        (h = ensure(B.snap, snap_words * sizeof(u64))) != hipSuccess)
      return hip_fail(e, h, "allocation");
    ctl1 = dp<MceCtl>(B.ctl1);
    if ((h = mce_launch_zero(dp<u64>(B.ctl1), sizeof(MceCtl) / sizeof(u64), s)) != hipSuccess ||
        (h = mce_launch_zero(dp<u64>(B.snap), snap_words, s)) != hipSuccess)
      return hip_fail(e, h, "clear");
  }
  if ((h = mce_launch_peel(n, row_ptr, col_idx, dp<int>(B.deg), dp<int>(B.rnd), dp<int>(B.core),
                           dp<int>(B.alive0), dp<int>(B.alive1), dp<int>(B.front0), dp<int>(B.front1),
                           dp<int>(B.bfront0), dp<int>(B.bfront1), ctl, budget,
                           tcap ? dp<unsigned short>(B.tcol) : nullptr, tcap, tcap ? dp<int>(B.tcrow) : nullptr,
                           pblocks, split ? 1 : 0, split ? dp<unsigned char>(B.snap) : nullptr,
                           split ? e->handed_ev : nullptr, s)) != hipSuccess)
    return hip_fail(e, h, "peel launch");
  if (timing) (void)hipEventRecord(e->ev[2], s);
  if (maxhubs > 0 && (h = mce_launch_hubs(n, row_ptr, col_idx, dp<int>(B.hub_id), dp<int>(B.hub_v),
                                         dp<u64>(B.hub_bm), maxhubs, ctl, grid, s)) != hipSuccess)
    return hip_fail(e, h, "hub bitmaps launch");
  // A first-level run over every vertex builds the forward adjacency before
  // the orientation, which then reads |P| from it; other runs build it after
  // the root bucketing when a build needs it (not mce_run_static: its scratch
  // has no room for nnz more entries).
  const bool early_fadj = !stat && !l2 && !subset;
  char* hio = stat ? reinterpret_cast<char*>(e->host_io) : static_cast<char*>(e->host.p);
  MceCtl* hctl = reinterpret_cast<MceCtl*>(hio);

  // Split peel: the search takes the hand-over order, set up on side stream 0
  // from the grid's hand-over event while the tail runs on s: its ranks, its
  // forward adjacency and the orientation of every root, read back; the whole
  // search is then planned from them. A return on any path after this waits
  // for that stream first.
  struct StreamGuard {
    hipStream_t st = nullptr;
    ~StreamGuard() {
      if (st) (void)hipStreamSynchronize(st);
    }
  } early_guard;
  hipStream_t es = e->side[0];
  bool handover = false;
  MceCtl* h1 = static_cast<MceCtl*>(e->host1.p);
  if (split) {
    if ((h = ensure(B.srank, (size_t)n * sizeof(int))) != hipSuccess ||
        (h = ensure(B.fadj1, (size_t)std::max<int64_t>(nnz, 1) * sizeof(int))) != hipSuccess ||
        (h = ensure(B.fdeg1, (size_t)n * sizeof(int))) != hipSuccess ||
        (h = ensure(B.flong1, (size_t)n * sizeof(int))) != hipSuccess ||
        (h = ensure(B.pcount1, (size_t)n * sizeof(int))) != hipSuccess ||
        (h = ensure(B.xcount1, (size_t)n * sizeof(int))) != hipSuccess ||
        (h = ensure_host(e->host1, sizeof(MceCtl))) != hipSuccess)
      return hip_fail(e, h, "allocation");
    h1 = static_cast<MceCtl*>(e->host1.p);
    early_guard.st = es;
    if ((h = hipStreamWaitEvent(es, e->handed_ev, 0)) != hipSuccess ||
        (h = mce_launch_search_rank(n, dp<int>(B.rnd), dp<int>(B.deg), dp<unsigned char>(B.snap), ctl,
                                    dp<int>(B.srank), grid, es)) != hipSuccess ||
        (h = mce_launch_forward_adj(n, row_ptr, col_idx, dp<int>(B.srank), dp<int>(B.fadj1), dp<int>(B.fdeg1),
                                    dp<int>(B.flong1), ctl1, e->num_cu * 16, es, ctl)) != hipSuccess ||
        (h = mce_launch_orient_handover(n, row_ptr, dp<int>(B.fdeg1), ctl, dp<int>(B.pcount1),
                                        dp<int>(B.xcount1), ctl1, grid, es)) != hipSuccess ||
        (h = hipMemcpyAsync(h1, ctl1, sizeof(MceCtl), hipMemcpyDeviceToHost, es)) != hipSuccess ||
        (h = hipStreamSynchronize(es)) != hipSuccess)
      return hip_fail(e, h, "hand-over orientation");
    // (a root of more than MCE_MAX_P later neighbours in the hand-over order:
    // the search waits for the peel's order instead, which may have none)
    handover = h1->tail_go != 0 && (h1->status & MCE_E_LIMIT) == 0;
  }
  if (!handover) {
    if (early_fadj &&
        ((h = take(arena, B.fadj, (size_t)std::max<int64_t>(nnz, 1) * sizeof(int))) != hipSuccess ||
         (h = take(arena, B.fdeg, (size_t)n * sizeof(int))) != hipSuccess ||
         (h = take(arena, B.flong, (size_t)n * sizeof(int))) != hipSuccess))
      return alloc_fail(e, arena, h, "forward adjacency");
    if (early_fadj && (h = mce_launch_forward_adj(n, row_ptr, col_idx, dp<int>(B.rnd), dp<int>(B.fadj),
                                                  dp<int>(B.fdeg), dp<int>(B.flong), ctl, e->num_cu * 16, s)) !=
                          hipSuccess)
      return hip_fail(e, h, "forward adjacency launch");
    if ((h = mce_launch_orient(n, row_ptr, col_idx, dp<int>(B.rnd), subset ? roots : nullptr, cnt,
                               dp<int>(B.pcount), dp<int>(B.xcount), ctl, l2 ? dp<u64>(B.fwd) : nullptr,
                               early_fadj ? dp<int>(B.fdeg) : nullptr, grid, s)) != hipSuccess)
      return hip_fail(e, h, "orient launch");
    if (l2 && (h = mce_launch_l2_roots(n, nnz, row_ptr, col_idx, dp<int>(B.rnd), subset ? roots : nullptr, cnt,
                                       dp<u64>(B.fwd), dp<u64>(B.fwdtmp), dp<int>(B.src), dp<int>(B.eroots),
                                       dp<int>(B.pcount2), dp<int>(B.xcount2), dp<int>(B.hub_id),
                                       dp<int>(B.hub_v), dp<u64>(B.hub_bm), maxhubs, ctl, grid, s)) != hipSuccess)
      return hip_fail(e, h, "second-level roots launch");
    if ((h = hipMemcpyAsync(hctl, ctl, sizeof(MceCtl), hipMemcpyDeviceToHost, s)) != hipSuccess)
      return hip_fail(e, h, "readback");
    if ((h = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, h, "synchronize after orient");
    const u32 gbits = hctl->status & 0x1Fu;
    e->info.max_degree = hctl->max_degree;
    if (gbits) {
      e->info.graph_errors = gbits;
      return fail(e, MCE_ERR_GRAPH, "input is not a simple undirected graph in CSR form");
    }
    if (hctl->status & MCE_E_TIMEOUT) return fail(e, MCE_ERR_TIMEOUT, "k-core peel ran past the time limit");
    if (hctl->status & MCE_E_ROOTS) return fail(e, MCE_ERR_ARG, "a root id is outside [0, n)");
    e->info.degeneracy = hctl->degeneracy;
    e->info.rounds = hctl->rounds;
    e->have_order = true;
  } else {
    // (the grid ran, so the input passed validation; the peel's order is known
    // once the tail ends, at the final read-back)
    e->info.max_degree = h1->max_degree;
  }
  // The facts the plan reads, the device control block whose cursors the
  // bucketing takes, the stream the plan's set-up runs on (it forks from it),
  // the order the builds split each root's neighbours by, the forward adjacency
  // and the roots' |P| and |X|: the hand-over order's or the peel's.
  const MceCtl* tc = handover ? h1 : hctl;
  MceCtl* tdev = handover ? ctl1 : ctl;
  hipStream_t fs = handover ? es : s;
  int* srnd = handover ? dp<int>(B.srank) : dp<int>(B.rnd);
  int* fadj_p = handover ? dp<int>(B.fadj1) : nullptr;
  int* fdeg_p = handover ? dp<int>(B.fdeg1) : nullptr;
  e->info.max_p = tc->max_p;
  e->info.max_x = tc->max_x;
  e->info.isolated = (int64_t)tc->isolated;
  if (tc->status & MCE_E_LIMIT)
    return fail(e, MCE_ERR_LIMIT, l2 ? "a second-level subtree has more than 2048 common later neighbours"
                                     : "a first-level subtree has more than 2048 later neighbours");
  // the subtree roots the search takes: vertex roots, or their forward edges
  const int nsub = l2 ? hctl->l2_roots : cnt;
  const int32_t* sroots = l2 ? dp<int>(B.eroots) : (subset ? roots : nullptr);
  int* spc = handover ? dp<int>(B.pcount1) : l2 ? dp<int>(B.pcount2) : dp<int>(B.pcount);
  int* sxc = handover ? dp<int>(B.xcount1) : l2 ? dp<int>(B.xcount2) : dp<int>(B.xcount);
  e->info.roots = nsub;

  // Induced-subgraph mode (section 3.4; section 4.5 picks partial when
  // Delta / d > 200, else full; with the hand-over order, d is the level the
  // peel had reached, a lower bound). Local row indices of the full subgraph
  // must stay below 2^20 for the pivot keys.
  int mode;
  const int dd = std::max(1, tc->degeneracy);
  const bool full_fits = (long long)tc->max_p + tc->max_x < (long long)MCE_MAX_LOCAL;
  if (e->cfg.subgraph == MCE_SUBGRAPH_PARTIAL) {
    mode = MCE_MODE_IP;
  } else if (e->cfg.subgraph == MCE_SUBGRAPH_FULL) {
    if (!full_fits) return fail(e, MCE_ERR_LIMIT, "full induced subgraph: |P| + |X| of a root exceeds 2^20");
    mode = MCE_MODE_IPX;
  } else {
    mode = (tc->max_degree > 200LL * dd || !full_fits) ? MCE_MODE_IP : MCE_MODE_IPX;
  }
  e->info.subgraph = mode == MCE_MODE_IPX ? MCE_SUBGRAPH_FULL : MCE_SUBGRAPH_PARTIAL;

  // roots per sub-class of that mode (and with the micro sub-class on or off)
  const int var = mode | (micro_on ? 0 : 2);
  SubOffsets off{};
  int counts[MCE_NSUB];
  int total = 0;
  size_t heap_words = 0;            // in series: the largest sub-class's tables; overlapped: all of them
  size_t heap_base[MCE_NSUB] = {};  // a sub-class's region (overlapped)
  for (int c = 0; c < MCE_NSUB; c++) {
    counts[c] = tc->sub_count[var][c];
    off.off[c] = total;
    total += counts[c];
    if (overlap) {
      heap_base[c] = heap_words;
      heap_words += (size_t)tc->sub_words[var][c];
    } else {
      heap_words = std::max(heap_words, (size_t)tc->sub_words[var][c]);
    }
  }
  const u64 iso = tc->isolated, iso_hash = tc->isolated_hash;

  // launch plan, heaviest width first; every buffer sized before any launch
  struct Plan {
    int sub, nw;
    size_t slot_off;   // its wavefront slots in B.slots (bytes)
    SearchLayout L;
  };
  Plan plan[MCE_NSUB];
  int nplan = 0;
  size_t slot_bytes = 0;
  int micro_nw = 0;
  int stat_rows = 0;
  const bool counters = (e->cfg.flags & MCE_FLAG_COUNTERS) != 0;
  int busy_subs = 0;   // sub-classes with roots: their launches
  for (int c = 0; c < MCE_NSUB; c++) busy_subs += counts[c] > 0 ? 1 : 0;
  for (int c = MCE_NSUB - 1; c >= 0; c--) {
    if (counts[c] == 0) continue;
    Plan pl{};
    pl.sub = c;
    int nw;
    if (c == MCE_SUB_MICRO) {
      nw = occupancy(e, -1 - (counters ? 1 : 0), 0LL, [&] { return mce_micro_max_workers(counters, e->num_cu); });
      nw = std::min(nw, (overlap && busy_subs > 1 ? MCE_MICRO_WAVES_PER_CU_BESIDE : MCE_MICRO_WAVES_PER_CU) *
                            e->num_cu);
    } else {
      pl.L = mce_search_layout(c, mode, tc->sub_maxp[var][c], tc->sub_maxx[var][c], tc->sub_maxr[var][c],
                               counts[c], e->num_cu, hbm, counters);
      const SearchLayout& L = pl.L;
      nw = occupancy(e, (((c * 2 + mode) * 2 + (counters ? 1 : 0)) * 2 + (L.srows ? 1 : 0)) * 2 + (L.sprows ? 1 : 0),
                     (long long)L.lds_bytes * 2 + (L.sstack ? 1 : 0),
                     [&] { return mce_search_max_workers(L, e->num_cu); });
    }
    if (nw <= 0) return fail(e, MCE_ERR_DEVICE, "search kernel occupancy query failed");
    if (c != MCE_SUB_MICRO && (c >> 1) == 0)
      nw = std::min(nw, (overlap && busy_subs > 1 ? kW1WavesPerCuBeside : kW1WavesPerCu) * e->num_cu);
    if (kWideWavesPerCu > 0 && overlap && busy_subs > 1 && c != MCE_SUB_MICRO && (c >> 1) > 0)
      nw = std::min(nw, kWideWavesPerCu * e->num_cu);
    if (e->cfg.max_workers > 0) nw = std::min(nw, (int)e->cfg.max_workers);
    if (!e->cfg.worker_list) nw = std::min(nw, counts[c]);
    pl.nw = nw;
    if (c == MCE_SUB_MICRO) {
      micro_nw = nw;
    } else if (overlap) {
      pl.slot_off = slot_bytes;
      slot_bytes += (pl.L.slot_bytes * (size_t)nw + 255) & ~(size_t)255;
    } else {
      slot_bytes = std::max(slot_bytes, pl.L.slot_bytes * (size_t)nw);
    }
    stat_rows += nw;
    plan[nplan++] = pl;
  }
  // the forward adjacency pays where a build reads rows of X members: micro
  // tables, and full-subgraph tables
  bool use_fadj = false;
  for (int i = 0; i < nplan; i++) use_fadj |= plan[i].sub == MCE_SUB_MICRO || mode == MCE_MODE_IPX;
  use_fadj = early_fadj || (use_fadj && !stat);
  // micro frame stacks: kMicroStack frames per wave; in the static scratch,
  // the largest power of two that the space left holds, at least
  // kMicroStackMinStatic (an overflow at run time is MCE_ERR_LIMIT)
  int micro_cap = stat ? kMicroStack : e->micro_stack;
  if (total > 0) {
    const size_t mail_bytes = (size_t)std::max(micro_nw, 1) * mce_micro_mail_words() * sizeof(u64);
    if ((h = take(arena, B.taboff, (size_t)total * sizeof(u64))) != hipSuccess ||
        (h = take(arena, B.scan, (size_t)mce_scan_temp_words(total) * sizeof(u64))) != hipSuccess ||
        (h = take(arena, B.heap, heap_words * sizeof(u64))) != hipSuccess ||
        (h = take(arena, B.slots, slot_bytes)) != hipSuccess ||
        (h = take(arena, B.stats, (size_t)stat_rows * MCE_NSTAT * sizeof(u64))) != hipSuccess ||
        (micro_nw && (h = take(arena, B.mail, mail_bytes)) != hipSuccess))
      return alloc_fail(e, arena, h, "search buffers");
    // the forward adjacency, for micro tables and the X rows of full-subgraph
    // tables (the builds read CSR rows otherwise: the static scratch has no
    // room for nnz more entries)
    if (use_fadj && !early_fadj &&
        ((h = take(arena, B.fadj, (size_t)std::max<int64_t>(nnz, 1) * sizeof(int))) != hipSuccess ||
         (h = take(arena, B.fdeg, (size_t)n * sizeof(int))) != hipSuccess ||
         (h = take(arena, B.flong, (size_t)n * sizeof(int))) != hipSuccess))
      return alloc_fail(e, arena, h, "forward adjacency");
    if (micro_nw) {
      const size_t frame_bytes = 6 * sizeof(u64) * (size_t)micro_nw;
      if (stat) {
        const size_t used = (arena.used + 255) & ~(size_t)255;
        const size_t room = arena.cap > used ? (arena.cap - used) / frame_bytes : 0;
        while (micro_cap > kMicroStackMinStatic && (size_t)micro_cap > room) micro_cap >>= 1;
      }
      if ((h = take(arena, B.mstack, frame_bytes * (size_t)micro_cap)) != hipSuccess)
        return alloc_fail(e, arena, h, "micro search stacks");
    }
    if ((h = mce_launch_bucket(sroots, nsub, spc, sxc, mode,
                               micro_on ? 1 : 0, off, dp<int>(B.lists), dp<u64>(B.taboff), tdev, grid, fs)) !=
        hipSuccess)
      return hip_fail(e, h, "bucket launch");
    // table sizes -> heap offsets (every sub-class's launch reuses the heap from its first root's offset)
    if ((h = mce_launch_scan(dp<u64>(B.taboff), total, dp<u64>(B.scan), fs)) != hipSuccess)
      return hip_fail(e, h, "table offset scan");
    if (use_fadj && !early_fadj && (h = mce_launch_forward_adj(n, row_ptr, col_idx, dp<int>(B.rnd), dp<int>(B.fadj),
                                                dp<int>(B.fdeg), dp<int>(B.flong), ctl, e->num_cu * 16, s)) != hipSuccess)
      return hip_fail(e, h, "forward adjacency launch");
  }
  if (!handover) {
    fadj_p = dp<int>(B.fadj);
    fdeg_p = dp<int>(B.fdeg);
  }
  if (timing) (void)hipEventRecord(e->ev[3], fs);

  // Overlapped: launch pi (its build, worker-list init and search) runs on side
  // stream pi mod MCE_SIDE_STREAMS, after everything queued so far on the
  // stream the set-up ran on, and s waits for every side stream used before the
  // read-back.
  bool side_used[MCE_SIDE_STREAMS] = {};
  bool side_forked[MCE_SIDE_STREAMS] = {};
  // with the hand-over order (set up on side stream 0): the launch with the
  // most table words (the longest chain) gets side stream 1 to itself, the
  // micro launch follows the set-up on side stream 0, and the other (short)
  // launches run one after another on side stream 2, where their builds come
  // before the long searches fill the compute units (three side streams, so
  // that with the caller's stream no two share a hardware queue; the micro
  // launch and the short ones taking streams 2 and 0 in turn: 17.8 against
  // 17.2 ms a step)
  if (handover) side_used[0] = true;
  int heavy = -1;
  if (handover) {
    u64 best = 0;
    for (int i = 0; i < nplan; i++) {
      const u64 w = tc->sub_words[var][plan[i].sub];
      if (plan[i].sub != MCE_SUB_MICRO && w >= best) {
        best = w;
        heavy = i;
      }
    }
  }
  auto launch_fail = [&](hipError_t herr, const char* what) {
    if (overlap)   // leave no launch of this run behind on a side stream
      for (int k = 0; k < MCE_SIDE_STREAMS; k++)
        if (side_used[k]) (void)hipStreamSynchronize(e->side[k]);
    return hip_fail(e, herr, what);
  };
  // overlapped: every launch's worker list is set up here, before the fork (a
  // small kernel queued behind a build on a busy side stream waits for free
  // compute units, and the search behind it waits too)
  if (overlap) {
    for (int pi = 0, so = 0; pi < nplan; pi++) {
      if ((h = mce_launch_wl_init(dp<MceWl>(B.wl) + pi, plan[pi].nw, dp<u64>(B.stats) + (size_t)so * MCE_NSTAT,
                                  fs)) != hipSuccess)
        return hip_fail(e, h, "wl init");
      so += plan[pi].nw;
    }
  }
  if (overlap && nplan > 0 && (h = hipEventRecord(e->fork_ev, fs)) != hipSuccess) return hip_fail(e, h, "fork");

  int launches = 0, max_workers_used = 0, stat_off = 0;
  int evi = 4;
  for (int pi = 0; pi < nplan; pi++) {
    const Plan& pl = plan[pi];
    const int c = pl.sub;
    const SearchLayout& L = pl.L;
    hipStream_t ls = s;
    if (overlap) {
      int k = pi % MCE_SIDE_STREAMS;
      if (handover) k = pi == heavy ? 1 : (c == MCE_SUB_MICRO ? 0 : 2);
      ls = e->side[k];
      if (!side_forked[k]) {
        if ((h = hipStreamWaitEvent(ls, e->fork_ev, 0)) != hipSuccess) return launch_fail(h, "fork");
        side_forked[k] = true;
        side_used[k] = true;
      }
    }
    u64* heap = dp<u64>(B.heap) + heap_base[c];
    const size_t hwords = overlap ? (size_t)tc->sub_words[var][c] : heap_words;
    MceWl* wl = dp<MceWl>(B.wl) + (overlap ? pi : 0);
    BuildParams bp{};
    bp.rp = row_ptr;
    bp.ci = col_idx;
    bp.rnd = srnd;
    bp.roots = dp<int>(B.lists) + off.off[c];
    bp.nroots = counts[c];
    const bool micro = c == MCE_SUB_MICRO;
    bp.W = micro ? 1 : 1 << L.wclass;
    bp.mode = micro ? MCE_MODE_IPX : mode;
    bp.micro = micro ? 1 : 0;
    bp.heap = heap;
    bp.heap_words = hwords;
    bp.tab_off = dp<u64>(B.taboff) + off.off[c];
    bp.status = &ctl->status;
    bp.l2 = l2 ? 1 : 0;
    bp.src = dp<int>(B.src);
    bp.hub_id = maxhubs > 0 ? dp<int>(B.hub_id) : nullptr;
    bp.hub_bm = dp<u64>(B.hub_bm);
    bp.hub_words = (n + 63) / 64;
    if (!micro) {
      // enough (root, part) blocks to fill the chip, at most one part per 64-row
      // slab, and at most about 8 slabs of the largest table per part
      const int nslab = std::max(1, (hctl->sub_maxr[var][c] + 63) / 64);
      const int want = (kSplitBlocksPerCu * e->num_cu + counts[c] - 1) / counts[c];
      bp.parts = std::max(1, std::min(std::max(want, (nslab + 7) / 8), nslab));
    }
    if (use_fadj) {   // (B.fadj may have been allocated after the peel: read the pointers here)
      bp.fadj = fadj_p;
      bp.fdeg = fdeg_p;
    }
    if (timing) (void)hipEventRecord(e->ev[evi], ls);
    if ((h = mce_launch_build(bp, e->num_cu * MCE_BUILD_BLOCKS_PER_CU, ls)) != hipSuccess)
      return launch_fail(h, "build launch");
    if (timing) (void)hipEventRecord(e->ev[evi + 1], ls);
    if (!overlap &&
        (h = mce_launch_wl_init(wl, pl.nw, dp<u64>(B.stats) + (size_t)stat_off * MCE_NSTAT, ls)) != hipSuccess)
      return launch_fail(h, "wl init");
    if (micro) {
      MicroParams mp{};
      mp.heap = heap;
      mp.tab_off = dp<u64>(B.taboff) + off.off[c];
      mp.nroots = counts[c];
      mp.nworkers = pl.nw;
      mp.stacks = dp<u64>(B.mstack);
      mp.stack_cap = micro_cap;
      mp.mail_words = mce_micro_mail_words();
      mp.mail = dp<u64>(B.mail);
      mp.g_hist = results + 1;
      mp.g_hash = results;
      mp.wl = wl;
      mp.donate_min_p = e->cfg.micro_donate_min_p > 0 ? (int)e->cfg.micro_donate_min_p : 10;
      mp.worker_list = e->cfg.worker_list ? 1 : 0;
      // Cooperative pivot scans pay when every wave works through its own
      // small roots; with few large roots they spread frames thinner over the
      // waves and cost steps (Moon-Moser n = 45: 271k -> 300k steps).
      mp.coop = counts[c] >= kMicroCoopRootsPerWave * pl.nw ? 1 : 0;
      mp.budget = budget;
      mp.t_run = &ctl->t_run;
      mp.status = &ctl->status;
      mp.stats = dp<u64>(B.stats) + (size_t)stat_off * MCE_NSTAT;
      mp.taken = &ctl->taken[launches];
      if (stimes) (void)hipEventRecord(e->ev[evi + 2], ls);
      if ((h = mce_launch_micro(counters, mp, ls)) != hipSuccess) return launch_fail(h, "micro search launch");
      if (stimes) (void)hipEventRecord(e->ev[evi + 3], ls);
      evi += 4;
      stat_off += pl.nw;
      launches++;
      max_workers_used = std::max(max_workers_used, pl.nw);
      continue;
    }
    SearchParams prm{};
    prm.rp = row_ptr;
    prm.ci = col_idx;
    prm.heap = heap;
    prm.tab_off = dp<u64>(B.taboff) + off.off[c];
    prm.nroots = counts[c];
    prm.nworkers = pl.nw;
    prm.hcap = L.hcap;
    prm.l_misc = L.l_misc;
    prm.l_hist = L.l_hist;
    prm.l_hv = L.l_hv;
    prm.l_pid = L.l_pid;
    prm.l_stack = L.l_stack;
    prm.l_rows = L.l_rows;
    prm.l_xx = L.l_xx;
    prm.slot_bytes = L.slot_bytes;
    prm.s_stack = L.s_stack;
    prm.s_xx = L.s_xx;
    prm.s_mail = L.s_mail;
    prm.g_hist = results + 1;
    prm.g_hash = results;
    prm.wl = wl;
    prm.slots = dp<char>(B.slots) + pl.slot_off;
    prm.donate_min_p = std::max(1, (int)e->cfg.donate_min_p);
    prm.worker_list = e->cfg.worker_list ? 1 : 0;
    prm.budget = budget;
    prm.t_run = &ctl->t_run;
    prm.status = &ctl->status;
    prm.stats = dp<u64>(B.stats) + (size_t)stat_off * MCE_NSTAT;
    prm.taken = &ctl->taken[launches];
    if (stimes) (void)hipEventRecord(e->ev[evi + 2], ls);
    if ((h = mce_launch_search(L, prm, ls)) != hipSuccess) return launch_fail(h, "search launch");
    if (stimes) (void)hipEventRecord(e->ev[evi + 3], ls);
    evi += 4;
    stat_off += pl.nw;
    launches++;
    max_workers_used = std::max(max_workers_used, pl.nw);
  }
  if (overlap) {
    for (int k = 0; k < MCE_SIDE_STREAMS; k++) {
      if (!side_used[k]) continue;
      if ((h = hipEventRecord(e->join_ev[k], e->side[k])) != hipSuccess ||
          (h = hipStreamWaitEvent(s, e->join_ev[k], 0)) != hipSuccess)
        return launch_fail(h, "join");
    }
  }
  // results: one read-back of the control block and the result words
  if ((h = hipMemcpyAsync(hio, ctl, kIoBytes, hipMemcpyDeviceToHost, s)) != hipSuccess)
    return hip_fail(e, h, "result readback");
  if ((h = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, h, "synchronize at end");
  const u64* hres = reinterpret_cast<const u64*>(hio + sizeof(MceCtl));
  if (handover) {   // the tail has ended: the peel's order is complete
    e->info.degeneracy = hctl->degeneracy;
    e->info.rounds = hctl->rounds;
    e->have_order = true;
  }
  if (hctl->status & MCE_E_PROTO) return fail(e, MCE_ERR_DEVICE, "worker-list bookkeeping error");
  if (hctl->status & MCE_E_LIMIT) return fail(e, MCE_ERR_LIMIT, "a subtree larger than its width class");
  if (hctl->status & MCE_E_MSTACK) {
    // the sums are of an aborted search: the caller runs again with larger stacks
    *grow = !stat && micro_cap < kMicroStackMax;
    return fail(e, MCE_ERR_LIMIT, "a micro frame stack (%d frames a wave) overflowed", micro_cap);
  }
  if (hctl->status & MCE_E_HEAP) return fail(e, MCE_ERR_DEVICE, "induced-subgraph heap overflow");

  uint64_t* hist = e->hist;
  for (size_t k = 0; k < kHistWords; k++) hist[k] = hres[1 + k];
  hist[1] += iso;
  hist[2] += hctl->pairs;   // second-level roots that are maximal cliques by themselves
  u64 count = 0;
  int32_t len = 0;
  for (size_t k = 0; k < kHistWords; k++) {
    count += hist[k];
    if (hist[k]) len = (int32_t)k + 1;
  }
  e->hist_len = len;
  e->count = count;
  e->hash = hres[0] + iso_hash + hctl->pairs_hash;
  e->have_result = true;
  // a search stopped at the time limit still reports the cliques it found
  // (every launch flushes what its waves found), marked incomplete
  e->complete = (hctl->status & MCE_E_TIMEOUT) == 0;
  e->info.complete = e->complete ? 1 : 0;
  {
    int64_t started = 0;
    for (int i = 0; i < launches; i++) started += std::min<int64_t>(hctl->taken[i], counts[plan[i].sub]);
    // roots that need no search: isolated vertices, and second-level roots that are cliques of size 2
    started += (int64_t)nsub - total;
    e->info.roots_started = started;
  }

  mce_run_stats& so = e->stats_out;
  so.workers = max_workers_used;
  so.launches = launches;
  so.handover_round = handover ? tc->tail_r0 : -1;
  u64 words_built = 0;
  for (int i = 0; i < nplan; i++) words_built += tc->sub_words[var][plan[i].sub];
  so.table_words = words_built;
  e->n_last_plan = nplan;
  for (int i = 0; i < nplan; i++) {
    e->last_plan[i] = {plan[i].sub, plan[i].nw, counts[plan[i].sub]};
    if (i < 16) {
      so.launch_sub[i] = plan[i].sub;
      so.launch_roots[i] = counts[plan[i].sub];
      so.launch_words[i] = tc->sub_words[var][plan[i].sub];
    }
  }
  for (int i = 0; i < 4; i++) so.peel_ticks[i] = hctl->peel_ticks[i];
  so.micro_roots = counts[MCE_SUB_MICRO];
  so.micro_stack_cap = micro_nw ? micro_cap : 0;
  e->last_stat_rows = stat_rows;
  e->last_timing = timing;
  e->last_stimes = stimes;
  e->stats_pending = true;
  if (e->complete && overlap && !l2 && !stat) {
    mce_engine::TableMap& tm = e->tabs;
    tm.mode = mode;
    tm.total = total;
    for (int c = 0; c < MCE_NSUB; c++) {
      tm.off[c] = off.off[c];
      tm.count[c] = counts[c];
      tm.heap_base[c] = heap_base[c];
    }
    tm.valid = true;
  }
  so.ms_total = ms_since(t0);
  if (!e->complete) return fail(e, MCE_ERR_TIMEOUT, "search ran past the time limit (results are partial)");
  return MCE_OK;
}

// A run: attempts until the micro kernel's frame stacks hold the search. No
// bound short of the whole tree caps a wavefront's stack (its 64 lanes share
// one LIFO stack, and a frame buried under newer ones stays there), so an
// overflow aborts the attempt, and the next one gets four times the frames.
// The engine keeps the grown size.
mce_status run_impl(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                    const int32_t* roots, int32_t nroots, bool subset, void* stream, Arena& arena) {
  for (;;) {
    bool grow = false;
    const mce_status st = run_once(e, n, nnz, row_ptr, col_idx, roots, nroots, subset, stream, arena, &grow);
    if (!grow) return st;
    e->micro_stack = std::min(kMicroStackMax, e->micro_stack * 4);
  }
}

// Per-wave counters and phase times of the last run, read on demand.
mce_status collect_stats(mce_engine* e) {
  if (!e->stats_pending) return MCE_OK;
  hipError_t h = hipSetDevice(e->device);
  if (h != hipSuccess) return hip_fail(e, h, "hipSetDevice");
  std::vector<u64> st((size_t)e->last_stat_rows * MCE_NSTAT);
  if (!st.empty() && (h = hipMemcpy(st.data(), e->last->stats.p, st.size() * sizeof(u64), hipMemcpyDeviceToHost)) !=
                         hipSuccess)
    return hip_fail(e, h, "stats readback");
  mce_run_stats& so = e->stats_out;
  std::vector<u64> stat_sum(MCE_NSTAT, 0);
  e->trace.clear();
  u64 max_busy = 0, max_nodes = 0, max_ticks = 0, start_spread = 0, max_stack = 0;
  int row = 0;
  for (int li = 0; li < e->n_last_plan; li++) {
    const auto& pl = e->last_plan[li];
    u64 smin = ~0ull, smax = 0;
    for (int w = 0; w < pl.nw; w++) {
      const u64* r = &st[(size_t)(row++) * MCE_NSTAT];
      mce_worker_record rec{};
      rec.launch = (int32_t)li;
      rec.worker = w;
      rec.start_tick = r[ST_START_ABS];
      rec.first_tick = r[ST_FIRST_ABS];
      rec.last_tick = r[ST_LAST_ABS];
      rec.end_tick = r[ST_START_ABS] + r[ST_TOTAL_TICKS];
      rec.busy_ticks = r[ST_BUSY_TICKS];
      rec.nodes = r[ST_NODES];
      rec.donations = r[ST_DONATIONS];
      rec.received = r[ST_RECEIVED];
      rec.hw_location = r[ST_HWID];
      rec.leaves = r[ST_LEAVES];
      rec.pivot_words = r[ST_PIVOT_WORDS];
      rec.branches = r[ST_BRANCHES];
      rec.xx_tests = r[ST_XX_TESTS];
      e->trace.push_back(rec);
      for (int i = 0; i < MCE_NSTAT; i++) stat_sum[i] += r[i];
      max_busy = std::max(max_busy, r[ST_BUSY_TICKS]);
      max_nodes = std::max(max_nodes, r[ST_NODES]);
      max_ticks = std::max(max_ticks, r[ST_TOTAL_TICKS]);
      max_stack = std::max(max_stack, r[ST_STACK_MAX]);
      if (r[ST_START_ABS]) {
        smin = std::min(smin, r[ST_START_ABS]);
        smax = std::max(smax, r[ST_START_ABS]);
      }
    }
    if (smax >= smin && smin != ~0ull) start_spread = std::max(start_spread, smax - smin);
  }
  so.nodes = stat_sum[ST_NODES];
  so.leaves = stat_sum[ST_LEAVES];
  so.donations = stat_sum[ST_DONATIONS];
  so.pivot_rows = stat_sum[ST_PIVOT_ROWS];
  so.pivot_words = stat_sum[ST_PIVOT_WORDS];
  so.xx_tests = stat_sum[ST_XX_TESTS];
  so.branches = stat_sum[ST_BRANCHES];
  so.busy_ticks = stat_sum[ST_BUSY_TICKS];
  so.max_busy_ticks = max_busy;
  so.max_nodes = max_nodes;
  so.kernel_ticks = max_ticks;
  so.donate_ticks = stat_sum[ST_DONATE_TICKS];
  so.setup_ticks = stat_sum[ST_SETUP_TICKS];
  so.first_ticks = stat_sum[ST_FIRST_TICKS];
  so.start_spread_ticks = start_spread;
  so.claim_checks = stat_sum[ST_CHECKS];
  so.donate_ok_ticks = stat_sum[ST_DONATE_OK_TICKS];
  so.max_stack_frames = max_stack;
  so.steps = stat_sum[ST_STEPS];
  so.lane_steps = stat_sum[ST_LANE_STEPS];
  static_assert(MCE_NACT == sizeof(so.act_cycles) / sizeof(so.act_cycles[0]), "activities");
  for (int i = 0; i < MCE_NACT; i++) so.act_cycles[i] = stat_sum[ST_ACT0 + i];
  if (e->last_timing) {
    float a = 0, b = 0, c = 0;
    (void)hipEventElapsedTime(&a, e->ev[0], e->ev[1]);
    (void)hipEventElapsedTime(&b, e->ev[1], e->ev[2]);
    (void)hipEventElapsedTime(&c, e->ev[2], e->ev[3]);
    so.ms_validate = a;
    so.ms_peel = b;
    so.ms_orient = c;   // orientation, host read-back and root bucketing
  }
  if (e->last_stimes) {
    double mb = 0, ms = 0;
    for (int i = 0; i < e->n_last_plan; i++) {
      float x = 0, y = 0;
      if (e->last_timing) (void)hipEventElapsedTime(&x, e->ev[4 + 4 * i], e->ev[5 + 4 * i]);
      (void)hipEventElapsedTime(&y, e->ev[6 + 4 * i], e->ev[7 + 4 * i]);
      mb += x;
      ms += y;
      if (i < 16) {
        so.launch_build_ms[i] = x;
        so.launch_search_ms[i] = y;
      }
    }
    so.ms_build = mb;
    so.ms_search = ms;
  }
  e->stats_pending = false;
  return MCE_OK;
}

}  // namespace

extern "C" {

mce_status mce_config_init(mce_config* cfg) {
  if (!cfg) return MCE_ERR_ARG;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->struct_size = sizeof(mce_config);
  cfg->device = -1;
  cfg->worker_list = 1;
  cfg->donate_min_p = 1;
  cfg->micro_donate_min_p = 10;
  cfg->validate = 1;
  cfg->max_workers = 0;
  cfg->timeout_ms = 120000;
  cfg->flags = 0;
  cfg->subgraph = MCE_SUBGRAPH_AUTO;
  return MCE_OK;
}

mce_status mce_create(const mce_config* cfg, mce_engine** out) {
  if (!out) return MCE_ERR_ARG;
  *out = nullptr;
  mce_config c;
  mce_config_init(&c);
  if (cfg) {
    size_t sz = cfg->struct_size ? std::min<size_t>(cfg->struct_size, sizeof(mce_config)) : sizeof(mce_config);
    std::memcpy(&c, cfg, sz);
    c.struct_size = sizeof(mce_config);
  }
  const bool stack_ok = c.micro_stack_frames == 0 ||
                        (c.micro_stack_frames >= 64 && c.micro_stack_frames <= (1 << 20) &&
                         (c.micro_stack_frames & (c.micro_stack_frames - 1)) == 0);
  if (!stack_ok || c.donate_min_p < 1 || c.micro_donate_min_p < 0 || c.max_workers < 0 || c.timeout_ms < 0 ||
      c.subgraph < MCE_SUBGRAPH_AUTO ||
      c.subgraph > MCE_SUBGRAPH_FULL ||
      (c.flags & ~(MCE_FLAG_HBM_STAGING | MCE_FLAG_PHASE_TIMES | MCE_FLAG_COUNTERS | MCE_FLAG_NO_MICRO |
                   MCE_FLAG_L2 | MCE_FLAG_SEARCH_TIMES | MCE_FLAG_SERIAL)) != 0)
    return MCE_ERR_ARG;
  if (c.timeout_ms == 0) c.timeout_ms = 120000;
  mce_engine* e = new (std::nothrow) mce_engine();
  if (!e) return MCE_ERR_NOMEM;
  e->cfg = c;
  e->micro_stack = c.micro_stack_frames ? c.micro_stack_frames : kMicroStack;
  int dev = c.device;
  if (dev < 0) {
    if (hipGetDevice(&dev) != hipSuccess) {
      delete e;
      return MCE_ERR_DEVICE;
    }
  }
  e->device = dev;
  if (hipSetDevice(dev) != hipSuccess) {
    delete e;
    return MCE_ERR_DEVICE;
  }
  int cus = 0, khz = 0, coop = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) {
    delete e;
    return MCE_ERR_DEVICE;
  }
  if (!coop) {
    delete e;
    return MCE_ERR_DEVICE;
  }
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
    e->tick_hz = (double)khz * 1e3;
  e->num_cu = cus;
  e->peel_blocks_max = mce_peel_max_blocks(cus);
  // the static scratch's device address, once per device, with the device current
  void* sp = nullptr;
  if (scratch_address(dev, &sp) != hipSuccess) {
    delete e;
    return MCE_ERR_DEVICE;
  }
  e->have_events = true;
  for (auto& ev : e->ev)
    if (hipEventCreate(&ev) != hipSuccess) e->have_events = false;
  bool side_ok = hipEventCreateWithFlags(&e->fork_ev, hipEventDisableTiming) == hipSuccess;
  for (int k = 0; k < MCE_SIDE_STREAMS; k++) {
    side_ok = side_ok && hipStreamCreateWithFlags(&e->side[k], hipStreamNonBlocking) == hipSuccess;
    side_ok = side_ok && hipEventCreateWithFlags(&e->join_ev[k], hipEventDisableTiming) == hipSuccess;
  }
  side_ok = side_ok && hipEventCreateWithFlags(&e->handed_ev, hipEventDisableTiming) == hipSuccess;
  if (!side_ok) {
    mce_destroy(e);
    return MCE_ERR_DEVICE;
  }
  *out = e;
  return MCE_OK;
}

mce_status mce_run(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                   void* stream) {
  Arena own;
  return run_impl(e, n, nnz, row_ptr, col_idx, nullptr, 0, false, stream, own);
}

mce_status mce_run_roots(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                         const int32_t* roots, int32_t nroots, void* stream) {
  Arena own;
  return run_impl(e, n, nnz, row_ptr, col_idx, roots, nroots, true, stream, own);
}

mce_status mce_run_static(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                          void* stream) {
  if (!e) return MCE_ERR_ARG;
  if (e->device < 0 || e->device >= kMaxDevices || !g_scratch_ptr[e->device])
    return fail(e, MCE_ERR_STATE, "the static scratch of device %d was not set up by mce_create", e->device);
  // one run at a time per process: every run on a device shares its scratch
  std::lock_guard<std::mutex> lk(g_static_run_mu);
  Arena a;
  a.base = static_cast<char*>(g_scratch_ptr[e->device]);
  a.cap = MCE_STATIC_SCRATCH_BYTES;
  return run_impl(e, n, nnz, row_ptr, col_idx, nullptr, 0, false, stream, a);
}

mce_status mce_result(const mce_engine* e, uint64_t* count, uint64_t* hash, uint64_t* hist, int32_t hist_cap,
                      int32_t* hist_len) {
  if (!e) return MCE_ERR_ARG;
  if (!e->have_result) return MCE_ERR_STATE;
  int32_t len = e->hist_len;
  if (hist_len) *hist_len = len;
  if (count) *count = e->count;
  if (hash) *hash = e->hash;
  if (hist) {
    if (hist_cap < len) return MCE_ERR_ARG;
    for (int32_t i = 0; i < len; i++) hist[i] = e->hist[i];
  }
  return e->complete ? MCE_OK : MCE_ERR_TIMEOUT;
}

mce_status mce_graph_info(const mce_engine* e, mce_graph_facts* info) {
  if (!e || !info) return MCE_ERR_ARG;
  *info = e->info;
  return MCE_OK;
}

mce_status mce_root_table(const mce_engine* e, int32_t root, uint64_t* words, int64_t cap, int64_t* len,
                          int32_t* form, void* stream) {
  if (!e || !len || !form || cap < 0 || (cap > 0 && !words)) return MCE_ERR_ARG;
  const mce_engine::TableMap& tm = e->tabs;
  if (!tm.valid || root < 0 || root >= e->last_n) return MCE_ERR_STATE;
  if (hipSetDevice(e->device) != hipSuccess) return MCE_ERR_DEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the root's place in the bucketed root lists, hence its sub-class
  std::vector<int32_t> lists((size_t)std::max(tm.total, 1));
  if (tm.total > 0 && (hipMemcpyAsync(lists.data(), e->own.lists.p, (size_t)tm.total * sizeof(int32_t),
                                      hipMemcpyDeviceToHost, s) != hipSuccess ||
                       hipStreamSynchronize(s) != hipSuccess))
    return MCE_ERR_DEVICE;
  int i = -1;
  for (int j = 0; j < tm.total; j++)
    if (lists[j] == root) {
      i = j;
      break;
    }
  if (i < 0) return MCE_ERR_STATE;   // no table: the root has no later neighbour
  int c = 0;
  while (c < MCE_NSUB && !(i >= tm.off[c] && i < tm.off[c] + tm.count[c])) c++;
  if (c == MCE_NSUB) return MCE_ERR_STATE;
  u64 to[2] = {0, 0};
  const u64* taboff = static_cast<const u64*>(e->own.taboff.p);
  if (hipMemcpyAsync(&to[0], taboff + i, sizeof(u64), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(&to[1], taboff + tm.off[c], sizeof(u64), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MCE_ERR_DEVICE;
  const u64* T = static_cast<const u64*>(e->own.heap.p) + tm.heap_base[c] + (to[0] - to[1]);
  u64 hdr = 0;
  if (hipMemcpyAsync(&hdr, T, sizeof(u64), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MCE_ERR_DEVICE;
  const int p = (int)(u32)hdr, x = (int)(hdr >> 32);
  const bool micro = c == MCE_SUB_MICRO;
  const int W = micro ? 1 : 1 << (c >> 1);
  const u64 nw = micro ? mce_micro_table_words(p, x) : mce_table_words(p, x, W, tm.mode);
  *len = (int64_t)nw;
  *form = W | (micro ? 1 << 8 : 0) | ((micro || tm.mode == MCE_MODE_IPX) ? 1 << 9 : 0);
  if ((u64)cap < nw) return MCE_ERR_ARG;
  if (hipMemcpyAsync(words, T, nw * sizeof(u64), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MCE_ERR_DEVICE;
  return MCE_OK;
}

mce_status mce_ordering(const mce_engine* e, int32_t* core, int32_t* round, void* stream) {
  if (!e) return MCE_ERR_ARG;
  if (!e->have_order) return MCE_ERR_STATE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  size_t nb = (size_t)e->last_n * sizeof(int32_t);
  if (nb == 0) return MCE_OK;
  if (hipSetDevice(e->device) != hipSuccess) return MCE_ERR_DEVICE;
  if (core && hipMemcpyAsync(core, e->last->core.p, nb, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MCE_ERR_DEVICE;
  if (round && hipMemcpyAsync(round, e->last->rnd.p, nb, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return MCE_ERR_DEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return MCE_ERR_DEVICE;
  return MCE_OK;
}

mce_status mce_stats(const mce_engine* e, mce_run_stats* stats) {
  if (!e || !stats) return MCE_ERR_ARG;
  const mce_status cs = collect_stats(const_cast<mce_engine*>(e));
  if (cs != MCE_OK) return cs;
  uint32_t want = stats->struct_size ? stats->struct_size : (uint32_t)sizeof(mce_run_stats);
  size_t n = std::min<size_t>(want, sizeof(mce_run_stats));
  std::memcpy(stats, &e->stats_out, n);
  stats->struct_size = (uint32_t)n;
  return MCE_OK;
}

mce_status mce_worker_trace(const mce_engine* e, mce_worker_record* out, int32_t cap, int32_t* count) {
  if (!e || cap < 0) return MCE_ERR_ARG;
  if (!e->have_result) return MCE_ERR_STATE;
  const mce_status cs = collect_stats(const_cast<mce_engine*>(e));
  if (cs != MCE_OK) return cs;
  const int32_t n = (int32_t)e->trace.size();
  if (count) *count = n;
  if (out) {
    for (int32_t i = 0; i < std::min(n, cap); i++) out[i] = e->trace[i];
  }
  return MCE_OK;
}

const char* mce_last_error(const mce_engine* e) { return e ? e->err : "null engine"; }

const char* mce_status_string(mce_status s) {
  switch (s) {
    case MCE_OK: return "MCE_OK";
    case MCE_ERR_ARG: return "MCE_ERR_ARG";
    case MCE_ERR_GRAPH: return "MCE_ERR_GRAPH";
    case MCE_ERR_NOMEM: return "MCE_ERR_NOMEM";
    case MCE_ERR_DEVICE: return "MCE_ERR_DEVICE";
    case MCE_ERR_STATE: return "MCE_ERR_STATE";
    case MCE_ERR_TIMEOUT: return "MCE_ERR_TIMEOUT";
    case MCE_ERR_LIMIT: return "MCE_ERR_LIMIT";
  }
  return "MCE_ERR_UNKNOWN";
}

void mce_destroy(mce_engine* e) {
  if (!e) return;
  (void)hipSetDevice(e->device);
  Bufs& b = e->own;   // the carved set points into the static scratch: nothing to free
  DevBuf* bufs[] = {&b.ctl,    &b.deg,    &b.rnd,     &b.core,    &b.alive0, &b.alive1,  &b.front0, &b.front1,
                    &b.bfront0, &b.bfront1, &b.pcount, &b.xcount,  &b.lists,  &b.taboff,  &b.scan,   &b.heap,
                    &b.wl,     &b.slots,  &b.stats,   &b.mstack,  &b.mail,   &b.src,     &b.fwd,    &b.fwdtmp,
                    &b.eroots, &b.pcount2, &b.xcount2, &b.hub_id, &b.hub_v,  &b.hub_bm, &b.fadj, &b.fdeg, &b.flong,
                    &b.tcol,   &b.tcrow,  &b.ctl1,    &b.snap,    &b.fadj1,   &b.fdeg1,  &b.flong1,  &b.pcount1, &b.xcount1,
                    &b.srank};
  for (DevBuf* d : bufs) release(*d);
  if (e->host.p) (void)hipHostFree(e->host.p);
  if (e->host1.p) (void)hipHostFree(e->host1.p);
  for (auto& ev : e->ev)
    if (ev) (void)hipEventDestroy(ev);
  for (auto& ev : e->join_ev)
    if (ev) (void)hipEventDestroy(ev);
  if (e->fork_ev) (void)hipEventDestroy(e->fork_ev);
  if (e->handed_ev) (void)hipEventDestroy(e->handed_ev);
  for (auto& st : e->side)
    if (st) (void)hipStreamDestroy(st);
  delete e;
}

}  // extern "C"
