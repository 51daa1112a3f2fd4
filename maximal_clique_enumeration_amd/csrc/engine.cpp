// Host side of the engine: the C ABI declared in include/mce.h.
//
// One mce_run queues, on the caller's stream: CSR validation, the k-core peel
// (degeneracy order, "Parallelizing Maximal Clique Enumeration on GPUs" section
// 2.4), the per-root P/X split, then one persistent search launch per bitset
// width class (sections 3.1-3.5), and reads back count, histogram and hash.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <map>
#include <new>
#include <string>
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

}  // namespace

struct mce_engine {
  mce_config cfg;
  int device = 0;
  int num_cu = 0;
  double tick_hz = 100e6;
  int peel_blocks_max = 1;
  std::string err;

  DevBuf ctl, deg, rnd, core, alive0, alive1, front0, front1, bfront0, bfront1, pcount, xcount, lists, taboff, scan, heap, wl,
      slots, stats, mstack, mail;
  DevBuf src, fwd, fwdtmp, eroots, pcount2, xcount2;   // second-level subtrees
  DevBuf hub_id, hub_v, hub_bm;                       // their hub adjacency bitmaps
  HostPinned host;    // staging for device -> host copies
  hipEvent_t ev[4 + 4 * MCE_NSUB] = {};
  bool have_events = false;

  // last run
  bool have_result = false;
  bool have_order = false;
  int32_t last_n = 0;
  uint64_t count = 0, hash = 0;
  std::vector<uint64_t> hist;
  mce_graph_facts info{};
  mce_run_stats stats_out{};
  std::vector<mce_worker_record> trace;

  // per-wave counters of the last run stay on the device until mce_stats or
  // mce_worker_trace asks for them (they are diagnostics, not results)
  struct LaunchInfo {
    int sub, nw, roots;
  };
  std::vector<LaunchInfo> last_plan;
  int last_stat_rows = 0;
  bool stats_pending = false;
  bool last_timing = false;
  bool last_stimes = false;   // the search launches carry events (MCE_FLAG_SEARCH_TIMES or _PHASE_TIMES)
  // resident-wave counts per kernel variant (occupancy queries cost ~0.1 ms each)
  std::map<std::pair<int, long long>, int> occupancy;
};

namespace {

mce_status fail(mce_engine* e, mce_status s, const std::string& msg) {
  if (e) e->err = msg;
  return s;
}

mce_status hip_fail(mce_engine* e, hipError_t h, const char* what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(h);
  return fail(e, h == hipErrorOutOfMemory ? MCE_ERR_NOMEM : MCE_ERR_DEVICE, m);
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

constexpr size_t kHistWords = MCE_MAX_P + 3;   // global histogram entries (sizes up to 2 + MCE_MAX_P)
// control block, then the result words (hash, histogram): one clear, one read-back
constexpr size_t kIoBytes = sizeof(MceCtl) + (1 + kHistWords) * sizeof(u64);
static_assert(sizeof(MceCtl) % sizeof(u64) == 0, "results follow the control block");
constexpr int kMaxHubs = 1024;                 // second-level orientation: hub adjacency bitmaps, at most
constexpr size_t kHubBytes = 256ull << 20;     // this many, in at most this many bytes
constexpr int kMicroStack = 4096;              // frames per wavefront stack of the micro search
constexpr int kMicroCoopRootsPerWave = 4;     // micro launches with this many roots per wave share pivot scans
// Tables other than micro ones are built by the split build: a root's rows are
// dealt over several blocks, about this many (root, part) blocks per CU.
constexpr int kSplitBlocksPerCu = 16;

mce_status run_impl(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                    const int32_t* roots, int32_t nroots, bool subset, void* stream) {
  const auto t0 = std::chrono::steady_clock::now();
  if (!e) return MCE_ERR_ARG;
  e->err.clear();
  e->have_result = false;
  e->have_order = false;
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
  e->hist.clear();
  e->count = e->hash = 0;
  e->last_n = n;
  const int cnt = subset ? nroots : n;
  e->info.roots = cnt;
  if (n == 0) {
    if (subset && nroots > 0) return fail(e, MCE_ERR_ARG, "roots given for an empty graph");
    e->have_result = true;
    e->stats_out.ms_total = ms_since(t0);
    return MCE_OK;
  }
  const bool timing = (e->cfg.flags & MCE_FLAG_PHASE_TIMES) && e->have_events;
  // events around the search launches only (every recorded event costs the stream a few us)
  const bool stimes = (timing || (e->cfg.flags & MCE_FLAG_SEARCH_TIMES)) && e->have_events;
  const bool hbm = (e->cfg.flags & MCE_FLAG_HBM_STAGING) != 0;
  const u64 budget = (u64)((double)e->cfg.timeout_ms * 1e-3 * e->tick_hz);

  size_t nb = (size_t)n * sizeof(int);
  if ((h = ensure(e->ctl, kIoBytes)) != hipSuccess || (h = ensure(e->deg, nb)) != hipSuccess ||
      (h = ensure(e->rnd, nb)) != hipSuccess || (h = ensure(e->core, nb)) != hipSuccess ||
      (h = ensure(e->alive0, nb)) != hipSuccess || (h = ensure(e->alive1, nb)) != hipSuccess ||
      (h = ensure(e->front0, nb)) != hipSuccess || (h = ensure(e->front1, nb)) != hipSuccess ||
      (h = ensure(e->bfront0, nb)) != hipSuccess || (h = ensure(e->bfront1, nb)) != hipSuccess ||
      (h = ensure(e->pcount, (size_t)std::max(cnt, 1) * sizeof(int))) != hipSuccess ||
      (h = ensure(e->xcount, (size_t)std::max(cnt, 1) * sizeof(int))) != hipSuccess ||
      (h = ensure(e->lists, (size_t)std::max(cnt, 1) * sizeof(int))) != hipSuccess ||
      (h = ensure(e->wl, sizeof(MceWl))) != hipSuccess ||
      (h = ensure_host(e->host, kIoBytes)) != hipSuccess)
    return hip_fail(e, h, "allocation");
  // second-level subtrees (section 3.2): the roots are the vertex roots' forward edges
  const bool l2 = (e->cfg.flags & MCE_FLAG_L2) != 0;
  e->info.level = l2 ? 2 : 1;
  int maxhubs = 0;
  if (l2) {
    const size_t ne = (size_t)std::max<int64_t>(nnz, 1) * sizeof(int);
    if ((h = ensure(e->src, ne)) != hipSuccess || (h = ensure(e->eroots, ne)) != hipSuccess ||
        (h = ensure(e->pcount2, ne)) != hipSuccess || (h = ensure(e->xcount2, ne)) != hipSuccess ||
        (h = ensure(e->fwd, (size_t)std::max(cnt, 1) * sizeof(u64))) != hipSuccess ||
        (h = ensure(e->fwdtmp, (size_t)mce_scan_temp_words(std::max(cnt, 1)) * sizeof(u64))) != hipSuccess)
      return hip_fail(e, h, "allocation");
  }
  // hub adjacency bitmaps (second-level runs; first-level builds did not gain
  // from them): n bits each, at most kMaxHubs within kHubBytes
  if (l2) {
    const size_t hub_bytes = ((size_t)n + 63) / 64 * sizeof(u64);
    maxhubs = (int)std::min<size_t>(kMaxHubs, kHubBytes / std::max<size_t>(hub_bytes, 1));
    if (maxhubs > 0 &&
        ((h = ensure(e->hub_id, (size_t)n * sizeof(int))) != hipSuccess ||
         (h = ensure(e->hub_v, (size_t)maxhubs * sizeof(int))) != hipSuccess ||
         (h = ensure(e->hub_bm, (size_t)maxhubs * hub_bytes)) != hipSuccess))
      return hip_fail(e, h, "allocation");
  }

  MceCtl* ctl = dp<MceCtl>(e->ctl);
  u64* results = reinterpret_cast<u64*>(dp<char>(e->ctl) + sizeof(MceCtl));   // hash, then the histogram
  if ((h = hipMemsetAsync(ctl, 0, kIoBytes, s)) != hipSuccess) return hip_fail(e, h, "memset");

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
  if ((h = mce_launch_peel(n, row_ptr, col_idx, dp<int>(e->deg), dp<int>(e->rnd), dp<int>(e->core),
                           dp<int>(e->alive0), dp<int>(e->alive1), dp<int>(e->front0), dp<int>(e->front1),
                           dp<int>(e->bfront0), dp<int>(e->bfront1), ctl, budget, pblocks, s)) != hipSuccess)
    return hip_fail(e, h, "peel launch");
  if (timing) (void)hipEventRecord(e->ev[2], s);
  if (maxhubs > 0 && (h = mce_launch_hubs(n, row_ptr, col_idx, dp<int>(e->hub_id), dp<int>(e->hub_v),
                                         dp<u64>(e->hub_bm), maxhubs, ctl, grid, s)) != hipSuccess)
    return hip_fail(e, h, "hub bitmaps launch");
  if ((h = mce_launch_orient(n, row_ptr, col_idx, dp<int>(e->rnd), subset ? roots : nullptr, cnt,
                             dp<int>(e->pcount), dp<int>(e->xcount), ctl, l2 ? dp<u64>(e->fwd) : nullptr, grid,
                             s)) != hipSuccess)
    return hip_fail(e, h, "orient launch");
  if (l2 && (h = mce_launch_l2_roots(n, nnz, row_ptr, col_idx, dp<int>(e->rnd), subset ? roots : nullptr, cnt,
                                     dp<u64>(e->fwd), dp<u64>(e->fwdtmp), dp<int>(e->src), dp<int>(e->eroots),
                                     dp<int>(e->pcount2), dp<int>(e->xcount2), dp<int>(e->hub_id),
                                     dp<int>(e->hub_v), dp<u64>(e->hub_bm), maxhubs, ctl, grid, s)) != hipSuccess)
    return hip_fail(e, h, "second-level roots launch");
  MceCtl* hctl = static_cast<MceCtl*>(e->host.p);
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
  e->info.max_p = hctl->max_p;
  e->info.max_x = hctl->max_x;
  e->info.isolated = (int64_t)hctl->isolated;
  e->have_order = true;
  if (hctl->status & MCE_E_LIMIT)
    return fail(e, MCE_ERR_LIMIT, l2 ? "a second-level subtree has more than 2048 common later neighbours"
                                     : "a first-level subtree has more than 2048 later neighbours");
  // the subtree roots the search takes: vertex roots, or their forward edges
  const int nsub = l2 ? hctl->l2_roots : cnt;
  const int32_t* sroots = l2 ? dp<int>(e->eroots) : (subset ? roots : nullptr);
  int* spc = l2 ? dp<int>(e->pcount2) : dp<int>(e->pcount);
  int* sxc = l2 ? dp<int>(e->xcount2) : dp<int>(e->xcount);
  e->info.roots = nsub;
  if (l2 && (h = ensure(e->lists, (size_t)std::max(nsub, 1) * sizeof(int))) != hipSuccess)
    return hip_fail(e, h, "allocation");

  // Induced-subgraph mode (section 3.4; section 4.5 picks partial when
  // Delta / d > 200, else full). Local row indices of the full subgraph must
  // stay below 2^20 for the pivot keys.
  int mode;
  const int dd = std::max(1, hctl->degeneracy);
  const bool full_fits = (long long)hctl->max_p + hctl->max_x < (long long)MCE_MAX_LOCAL;
  if (e->cfg.subgraph == MCE_SUBGRAPH_PARTIAL) {
    mode = MCE_MODE_IP;
  } else if (e->cfg.subgraph == MCE_SUBGRAPH_FULL) {
    if (!full_fits) return fail(e, MCE_ERR_LIMIT, "full induced subgraph: |P| + |X| of a root exceeds 2^20");
    mode = MCE_MODE_IPX;
  } else {
    mode = (hctl->max_degree > 200LL * dd || !full_fits) ? MCE_MODE_IP : MCE_MODE_IPX;
  }
  e->info.subgraph = mode == MCE_MODE_IPX ? MCE_SUBGRAPH_FULL : MCE_SUBGRAPH_PARTIAL;

  // roots per sub-class of that mode (and with the micro sub-class on or off)
  const bool micro_on = (e->cfg.flags & MCE_FLAG_NO_MICRO) == 0;
  const int var = mode | (micro_on ? 0 : 2);
  SubOffsets off{};
  int counts[MCE_NSUB];
  int total = 0;
  size_t heap_words = 0;
  for (int c = 0; c < MCE_NSUB; c++) {
    counts[c] = hctl->sub_count[var][c];
    off.off[c] = total;
    total += counts[c];
    heap_words = std::max(heap_words, (size_t)hctl->sub_words[var][c]);
  }
  const u64 iso = hctl->isolated, iso_hash = hctl->isolated_hash;

  // launch plan, heaviest width first; every buffer sized before any launch
  struct Plan {
    int sub, nw;
    SearchLayout L;
  };
  std::vector<Plan> plan;
  size_t slot_bytes = 0, mstack_bytes = 0, mail_bytes = 0;
  int stat_rows = 0;
  const bool counters = (e->cfg.flags & MCE_FLAG_COUNTERS) != 0;
  for (int c = MCE_NSUB - 1; c >= 0; c--) {
    if (counts[c] == 0) continue;
    Plan pl{};
    pl.sub = c;
    int nw;
    if (c == MCE_SUB_MICRO) {
      // 8 wavefronts per CU: more add start-up spread and little throughput
      const auto key = std::make_pair(-1 - (counters ? 1 : 0), 0LL);
      auto it = e->occupancy.find(key);
      if (it == e->occupancy.end()) it = e->occupancy.emplace(key, mce_micro_max_workers(counters, e->num_cu)).first;
      nw = std::min(it->second, 8 * e->num_cu);
      mstack_bytes = (size_t)std::max(nw, 1) * 6 * kMicroStack * sizeof(u64);
      mail_bytes = (size_t)std::max(nw, 1) * mce_micro_mail_words() * sizeof(u64);
    } else {
      pl.L = mce_search_layout(c, mode, hctl->sub_maxp[var][c], hctl->sub_maxx[var][c], hctl->sub_maxr[var][c],
                               hbm, counters);
      const auto key = std::make_pair(((c * 2 + mode) * 2 + (counters ? 1 : 0)) * 2 + (pl.L.srows ? 1 : 0),
                                      (long long)pl.L.lds_bytes * 2 + (pl.L.sstack ? 1 : 0));
      auto it = e->occupancy.find(key);
      if (it == e->occupancy.end()) it = e->occupancy.emplace(key, mce_search_max_workers(pl.L, e->num_cu)).first;
      nw = it->second;
    }
    if (nw <= 0) return fail(e, MCE_ERR_DEVICE, "search kernel occupancy query failed");
    if (e->cfg.max_workers > 0) nw = std::min(nw, (int)e->cfg.max_workers);
    if (!e->cfg.worker_list) nw = std::min(nw, counts[c]);
    pl.nw = nw;
    if (c != MCE_SUB_MICRO) slot_bytes = std::max(slot_bytes, pl.L.slot_bytes * (size_t)nw);
    stat_rows += nw;
    plan.push_back(pl);
  }
  if (total > 0) {
    if ((h = ensure(e->taboff, (size_t)total * sizeof(u64))) != hipSuccess ||
        (h = ensure(e->scan, (size_t)mce_scan_temp_words(total) * sizeof(u64))) != hipSuccess ||
        (h = ensure(e->heap, heap_words * sizeof(u64))) != hipSuccess ||
        (h = ensure(e->slots, slot_bytes)) != hipSuccess ||
        (h = ensure(e->stats, (size_t)stat_rows * MCE_NSTAT * sizeof(u64))) != hipSuccess ||
        (mstack_bytes && (h = ensure(e->mstack, mstack_bytes)) != hipSuccess) ||
        (mail_bytes && (h = ensure(e->mail, mail_bytes)) != hipSuccess))
      return hip_fail(e, h, "search buffers");
    if ((h = mce_launch_bucket(sroots, nsub, spc, sxc, mode,
                               micro_on ? 1 : 0, off, dp<int>(e->lists), dp<u64>(e->taboff), ctl, grid, s)) !=
        hipSuccess)
      return hip_fail(e, h, "bucket launch");
    // table sizes -> heap offsets (every sub-class's launch reuses the heap from its first root's offset)
    if ((h = mce_launch_scan(dp<u64>(e->taboff), total, dp<u64>(e->scan), s)) != hipSuccess)
      return hip_fail(e, h, "table offset scan");
  }
  if (timing) (void)hipEventRecord(e->ev[3], s);

  int launches = 0, max_workers_used = 0, stat_off = 0;
  int evi = 4;
  for (const Plan& pl : plan) {
    const int c = pl.sub;
    const SearchLayout& L = pl.L;
    BuildParams bp{};
    bp.rp = row_ptr;
    bp.ci = col_idx;
    bp.rnd = dp<int>(e->rnd);
    bp.roots = dp<int>(e->lists) + off.off[c];
    bp.nroots = counts[c];
    const bool micro = c == MCE_SUB_MICRO;
    bp.W = micro ? 1 : 1 << L.wclass;
    bp.mode = micro ? MCE_MODE_IPX : mode;
    bp.micro = micro ? 1 : 0;
    bp.heap = dp<u64>(e->heap);
    bp.heap_words = heap_words;
    bp.tab_off = dp<u64>(e->taboff) + off.off[c];
    bp.status = &ctl->status;
    bp.l2 = l2 ? 1 : 0;
    bp.src = dp<int>(e->src);
    bp.hub_id = maxhubs > 0 ? dp<int>(e->hub_id) : nullptr;
    bp.hub_bm = dp<u64>(e->hub_bm);
    bp.hub_words = (n + 63) / 64;
    if (!micro) {
      // enough (root, part) blocks to fill the chip, at most one part per 64-row
      // slab, and at most about 8 slabs of the largest table per part
      const int nslab = std::max(1, (hctl->sub_maxr[var][c] + 63) / 64);
      const int want = (kSplitBlocksPerCu * e->num_cu + counts[c] - 1) / counts[c];
      bp.parts = std::max(1, std::min(std::max(want, (nslab + 7) / 8), nslab));
    }
    if (timing) (void)hipEventRecord(e->ev[evi], s);
    if ((h = mce_launch_build(bp, e->num_cu * 32, s)) != hipSuccess) return hip_fail(e, h, "build launch");
    if (timing) (void)hipEventRecord(e->ev[evi + 1], s);
    if ((h = mce_launch_wl_init(dp<MceWl>(e->wl), pl.nw, dp<u64>(e->stats) + (size_t)stat_off * MCE_NSTAT, s)) !=
        hipSuccess)
      return hip_fail(e, h, "wl init");
    if (micro) {
      MicroParams mp{};
      mp.heap = dp<u64>(e->heap);
      mp.tab_off = dp<u64>(e->taboff) + off.off[c];
      mp.nroots = counts[c];
      mp.nworkers = pl.nw;
      mp.stacks = dp<u64>(e->mstack);
      mp.stack_cap = kMicroStack;
      mp.mail_words = mce_micro_mail_words();
      mp.mail = dp<u64>(e->mail);
      mp.g_hist = results + 1;
      mp.g_hash = results;
      mp.wl = dp<MceWl>(e->wl);
      mp.donate_min_p = e->cfg.micro_donate_min_p > 0 ? (int)e->cfg.micro_donate_min_p : 10;
      mp.worker_list = e->cfg.worker_list ? 1 : 0;
      // Cooperative pivot scans pay when every wave works through its own
      // small roots; with few large roots they spread frames thinner over the
      // waves and cost steps (Moon-Moser n = 45: 271k -> 300k steps).
      mp.coop = counts[c] >= kMicroCoopRootsPerWave * pl.nw ? 1 : 0;
      mp.budget = budget;
      mp.t_run = &ctl->t_run;
      mp.status = &ctl->status;
      mp.stats = dp<u64>(e->stats) + (size_t)stat_off * MCE_NSTAT;
      if (stimes) (void)hipEventRecord(e->ev[evi + 2], s);
      if ((h = mce_launch_micro(counters, mp, s)) != hipSuccess) return hip_fail(e, h, "micro search launch");
      if (stimes) (void)hipEventRecord(e->ev[evi + 3], s);
      evi += 4;
      stat_off += pl.nw;
      launches++;
      max_workers_used = std::max(max_workers_used, pl.nw);
      continue;
    }
    SearchParams prm{};
    prm.rp = row_ptr;
    prm.ci = col_idx;
    prm.heap = dp<u64>(e->heap);
    prm.tab_off = dp<u64>(e->taboff) + off.off[c];
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
    prm.wl = dp<MceWl>(e->wl);
    prm.slots = dp<char>(e->slots);
    prm.donate_min_p = std::max(1, (int)e->cfg.donate_min_p);
    prm.worker_list = e->cfg.worker_list ? 1 : 0;
    prm.budget = budget;
    prm.t_run = &ctl->t_run;
    prm.status = &ctl->status;
    prm.stats = dp<u64>(e->stats) + (size_t)stat_off * MCE_NSTAT;
    if (stimes) (void)hipEventRecord(e->ev[evi + 2], s);
    if ((h = mce_launch_search(L, prm, s)) != hipSuccess) return hip_fail(e, h, "search launch");
    if (stimes) (void)hipEventRecord(e->ev[evi + 3], s);
    evi += 4;
    stat_off += pl.nw;
    launches++;
    max_workers_used = std::max(max_workers_used, pl.nw);
  }
  // results: one read-back of the control block and the result words
  if ((h = hipMemcpyAsync(e->host.p, ctl, kIoBytes, hipMemcpyDeviceToHost, s)) != hipSuccess)
    return hip_fail(e, h, "result readback");
  if ((h = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, h, "synchronize at end");
  const u64* hres = reinterpret_cast<const u64*>(static_cast<const char*>(e->host.p) + sizeof(MceCtl));
  if (hctl->status & MCE_E_TIMEOUT) return fail(e, MCE_ERR_TIMEOUT, "search ran past the time limit");
  if (hctl->status & MCE_E_PROTO) return fail(e, MCE_ERR_DEVICE, "worker-list bookkeeping error");
  if (hctl->status & MCE_E_LIMIT) return fail(e, MCE_ERR_LIMIT, "subtree larger than its width class");
  if (hctl->status & MCE_E_HEAP) return fail(e, MCE_ERR_DEVICE, "induced-subgraph heap overflow");

  std::vector<uint64_t> hist(kHistWords, 0);
  for (size_t k = 0; k < kHistWords; k++) hist[k] = hres[1 + k];
  hist[1] += iso;
  hist[2] += hctl->pairs;   // second-level roots that are maximal cliques by themselves
  u64 count = 0;
  size_t len = 0;
  for (size_t k = 0; k < kHistWords; k++) {
    count += hist[k];
    if (hist[k]) len = k + 1;
  }
  hist.resize(len);
  e->hist = hist;
  e->count = count;
  e->hash = hres[0] + iso_hash + hctl->pairs_hash;
  e->have_result = true;

  mce_run_stats& so = e->stats_out;
  so.workers = max_workers_used;
  so.launches = launches;
  u64 words_built = 0;
  for (const Plan& pl : plan) words_built += hctl->sub_words[var][pl.sub];
  so.table_words = words_built;
  e->last_plan.clear();
  for (size_t i = 0; i < plan.size(); i++) {
    e->last_plan.push_back({plan[i].sub, plan[i].nw, counts[plan[i].sub]});
    if (i < 16) {
      so.launch_sub[i] = plan[i].sub;
      so.launch_roots[i] = counts[plan[i].sub];
    }
  }
  for (int i = 0; i < 4; i++) so.peel_ticks[i] = hctl->peel_ticks[i];
  so.micro_roots = counts[MCE_SUB_MICRO];
  e->last_stat_rows = stat_rows;
  e->last_timing = timing;
  e->last_stimes = stimes;
  e->stats_pending = true;
  so.ms_total = ms_since(t0);
  return MCE_OK;
}

// Per-wave counters and phase times of the last run, read on demand.
mce_status collect_stats(mce_engine* e) {
  if (!e->stats_pending) return MCE_OK;
  hipError_t h = hipSetDevice(e->device);
  if (h != hipSuccess) return hip_fail(e, h, "hipSetDevice");
  std::vector<u64> st((size_t)e->last_stat_rows * MCE_NSTAT);
  if (!st.empty() && (h = hipMemcpy(st.data(), e->stats.p, st.size() * sizeof(u64), hipMemcpyDeviceToHost)) !=
                         hipSuccess)
    return hip_fail(e, h, "stats readback");
  mce_run_stats& so = e->stats_out;
  std::vector<u64> stat_sum(MCE_NSTAT, 0);
  e->trace.clear();
  u64 max_busy = 0, max_nodes = 0, max_ticks = 0, start_spread = 0, max_stack = 0;
  int row = 0;
  for (size_t li = 0; li < e->last_plan.size(); li++) {
    const auto& pl = e->last_plan[li];
    u64 smin = ~0ull, smax = 0;
    for (int w = 0; w < pl.nw; w++, row++) {
      const u64* r = &st[(size_t)row * MCE_NSTAT];
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
    for (int i = 0; i < (int)e->last_plan.size(); i++) {
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
  if (c.donate_min_p < 1 || c.micro_donate_min_p < 0 || c.max_workers < 0 || c.timeout_ms < 0 ||
      c.subgraph < MCE_SUBGRAPH_AUTO ||
      c.subgraph > MCE_SUBGRAPH_FULL ||
      (c.flags & ~(MCE_FLAG_HBM_STAGING | MCE_FLAG_PHASE_TIMES | MCE_FLAG_COUNTERS | MCE_FLAG_NO_MICRO |
                   MCE_FLAG_L2 | MCE_FLAG_SEARCH_TIMES)) != 0)
    return MCE_ERR_ARG;
  if (c.timeout_ms == 0) c.timeout_ms = 120000;
  mce_engine* e = new (std::nothrow) mce_engine();
  if (!e) return MCE_ERR_NOMEM;
  e->cfg = c;
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
  e->have_events = true;
  for (auto& ev : e->ev)
    if (hipEventCreate(&ev) != hipSuccess) e->have_events = false;
  *out = e;
  return MCE_OK;
}

mce_status mce_run(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                   void* stream) {
  return run_impl(e, n, nnz, row_ptr, col_idx, nullptr, 0, false, stream);
}

mce_status mce_run_roots(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                         const int32_t* roots, int32_t nroots, void* stream) {
  return run_impl(e, n, nnz, row_ptr, col_idx, roots, nroots, true, stream);
}

mce_status mce_result(const mce_engine* e, uint64_t* count, uint64_t* hash, uint64_t* hist, int32_t hist_cap,
                      int32_t* hist_len) {
  if (!e) return MCE_ERR_ARG;
  if (!e->have_result) return MCE_ERR_STATE;
  int32_t len = (int32_t)e->hist.size();
  if (hist_len) *hist_len = len;
  if (count) *count = e->count;
  if (hash) *hash = e->hash;
  if (hist) {
    if (hist_cap < len) return MCE_ERR_ARG;
    for (int32_t i = 0; i < len; i++) hist[i] = e->hist[i];
  }
  return MCE_OK;
}

mce_status mce_graph_info(const mce_engine* e, mce_graph_facts* info) {
  if (!e || !info) return MCE_ERR_ARG;
  *info = e->info;
  return MCE_OK;
}

mce_status mce_ordering(const mce_engine* e, int32_t* core, int32_t* round, void* stream) {
  if (!e) return MCE_ERR_ARG;
  if (!e->have_order) return MCE_ERR_STATE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  size_t nb = (size_t)e->last_n * sizeof(int32_t);
  if (nb == 0) return MCE_OK;
  if (hipSetDevice(e->device) != hipSuccess) return MCE_ERR_DEVICE;
  if (core && hipMemcpyAsync(core, e->core.p, nb, hipMemcpyDeviceToDevice, s) != hipSuccess) return MCE_ERR_DEVICE;
  if (round && hipMemcpyAsync(round, e->rnd.p, nb, hipMemcpyDeviceToDevice, s) != hipSuccess) return MCE_ERR_DEVICE;
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

const char* mce_last_error(const mce_engine* e) { return e ? e->err.c_str() : "null engine"; }

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
  DevBuf* bufs[] = {&e->ctl,    &e->deg,   &e->rnd,    &e->core,    &e->alive0, &e->alive1,
                    &e->front0, &e->front1, &e->bfront0, &e->bfront1, &e->pcount, &e->xcount, &e->lists,  &e->taboff, &e->scan,
                    &e->heap,   &e->wl,    &e->slots,  &e->stats,  &e->mstack, &e->mail,
                    &e->src,    &e->fwd,   &e->fwdtmp, &e->eroots, &e->pcount2, &e->xcount2,
                    &e->hub_id, &e->hub_v, &e->hub_bm};
  for (DevBuf* b : bufs) release(*b);
  if (e->host.p) (void)hipHostFree(e->host.p);
  for (auto& ev : e->ev)
    if (ev) (void)hipEventDestroy(ev);
  delete e;
}

}  // extern "C"
