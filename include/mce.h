/*
 * mce.h -- C ABI of the MI355X (gfx950) maximal clique enumeration engine.
 *
 * The engine computes every maximal clique of a simple undirected graph exactly
 * ("Parallelizing Maximal Clique Enumeration on GPUs", arxiv 2212.01473v2,
 * section 2.1 states the problem; section 4.1 times the clique count together
 * with the degeneracy ordering). A clique C is maximal when no vertex outside C
 * is adjacent to every member of C. It returns three results instead of listing
 * cliques:
 *   - count: the number of maximal cliques (64-bit; section 4, Table 1 has graphs
 *     with more than 2^32 of them);
 *   - hist[k]: the number of maximal cliques with k vertices;
 *   - hash: an order-free 64-bit digest of the clique set,
 *         h(c)     = mix64(c + G)
 *         hash(C)  = mix64(sum_{c in C} h(c) + |C| * G)       (mod 2^64)
 *         hash     = sum over maximal cliques C of hash(C)    (mod 2^64)
 *     where c is an input vertex id, G = 0x9E3779B97F4A7C15 and mix64 is the
 *     SplitMix64 finaliser (Steele, Lea and Flood, OOPSLA 2014). The pages only
 *     count cliques; the digest exists so that two engines can be compared on
 *     the set itself.
 *
 * Method (all on the GPU): a k-core peel gives a degeneracy order (section 2.4);
 * every vertex roots an independent first-level subtree (section 2.4, Algorithm
 * 3) searched depth-first by one wavefront with Bron-Kerbosch pivoting (section
 * 2.3, Algorithm 2) over a bit-encoded partial or full induced subgraph (section
 * 3.4, built per root into device memory before the search) and a compact
 * excluded set (section 3.5); idle wavefronts receive branches from busy ones
 * through a worker list (section 3.3).
 *
 * Threading: an engine belongs to one host thread at a time. Engines are
 * independent of each other. Every call returns an mce_status; no call throws.
 */
#ifndef MCE_H
#define MCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mce_engine mce_engine;

typedef enum {
  MCE_OK = 0,
  MCE_ERR_ARG = -1,      /* bad argument: null pointer, negative size, buffer too small */
  MCE_ERR_GRAPH = -2,    /* input is not a simple undirected graph in CSR form */
  MCE_ERR_NOMEM = -3,    /* device or host allocation failed */
  MCE_ERR_DEVICE = -4,   /* a HIP runtime call failed */
  MCE_ERR_STATE = -5,    /* call out of order, e.g. mce_result before any run */
  MCE_ERR_TIMEOUT = -6,  /* the run passed mce_config.timeout_ms and was abandoned; if the search
                            had started, the cliques found before the limit are kept (see
                            mce_result and mce_graph_facts.complete) */
  MCE_ERR_LIMIT = -7     /* the graph exceeds a limit of this build (degeneracy > 2048), or a micro
                            frame stack overflowed at 2^20 frames (mce_run_static: at what its
                            scratch holds) */
} mce_status;

/* Classes of malformed input, reported in mce_graph_info.graph_errors when
   mce_run returns MCE_ERR_GRAPH (section 2.1: G is simple and undirected). */
#define MCE_GRAPH_ROWPTR 1u  /* row_ptr[0] != 0, row_ptr[n] != nnz, or a row that runs backwards */
#define MCE_GRAPH_RANGE 2u   /* a column id outside [0, n) */
#define MCE_GRAPH_LOOP 4u    /* a self-loop (v, v) */
#define MCE_GRAPH_ORDER 8u   /* a row not strictly ascending: unsorted or a duplicate edge */
#define MCE_GRAPH_ASYM 16u   /* u in N(v) but v not in N(u) */

/* mce_config.flags */
#define MCE_FLAG_HBM_STAGING 1u  /* keep induced-subgraph rows and DFS stacks in HBM even
                                    when they fit in LDS (section 3.4 data in device memory) */
#define MCE_FLAG_PHASE_TIMES 2u  /* record per-phase GPU times in mce_run_stats */
#define MCE_FLAG_COUNTERS 4u     /* count pivot rows, X_X tests and branches (mce_run_stats.pivot_rows,
                                    xx_tests, branches); the width-1 search kernel skips them otherwise */
#define MCE_FLAG_NO_MICRO 8u     /* subtrees with |P| <= 64 and |X| <= 64 go to the width-1 wavefront
                                    kernel like the rest; by default the micro kernel searches them, one
                                    search-tree node per lane (section 3.1's finer work split) */
#define MCE_FLAG_L2 16u          /* independent second-level subtrees (section 3.2, Algorithm 4): one
                                    subtree per edge {v, w}, w after v, with R = {v, w}, P = the common
                                    neighbours after w and X = those before w; a vertex of degree 0 is a
                                    clique of its own. The cliques found are the same; for mce_run_roots,
                                    the subtrees of the edges leaving the listed roots. By default one
                                    first-level subtree per vertex (Algorithm 3), which section 4.5
                                    recommends */

#define MCE_FLAG_SEARCH_TIMES 32u /* events around the search launches only (mce_run_stats.ms_search,
                                    launch_search_ms; the other phase times stay 0): the light form of
                                    MCE_FLAG_PHASE_TIMES for timing loops, since every recorded event
                                    costs the stream a few microseconds */
#define MCE_FLAG_SERIAL 64u      /* run the sub-class launches (build, then search) one after another on
                                    the caller's stream, reusing one table heap. By default each
                                    sub-class has its own heap region and its build and search run on
                                    one of the engine's own streams, forked from and joined back to the
                                    caller's stream, so that the launches overlap (a build, which waits
                                    on memory, beside another sub-class's search). mce_run_static always
                                    runs them in series. The results are the same either way. */
#define MCE_SIDE_STREAMS 4       /* the engine's own streams for the overlapped launches */

/* mce_config.subgraph: how each subtree's induced subgraph is encoded (section
   3.4). Partial: bit rows for P x P only, edges between P and X looked up in the
   CSR, pivot drawn from P u X_P (section 3.5, last paragraph). Full: bit rows for
   (P u X) x P, pivot drawn from all of P u X. Auto follows section 4.5: partial
   when Delta / d > 200, else full. */
#define MCE_SUBGRAPH_AUTO 0
#define MCE_SUBGRAPH_PARTIAL 1
#define MCE_SUBGRAPH_FULL 2

typedef struct {
  uint32_t struct_size;   /* sizeof(mce_config); 0 is taken as the current size */
  int32_t device;         /* HIP device ordinal; -1: the device current at mce_create */
  int32_t worker_list;    /* 1: idle wavefronts receive donated branches (section 3.3); 0: off */
  int32_t donate_min_p;   /* wavefront kernels: donate a branch only if its P has at least this
                             many vertices; must be >= 1. Section 3.3 uses 10; on power-law graphs
                             most shallow branches have fewer, and 10 kept nearly all work in the
                             wave that took the root (4M-vertex Chung-Lu sample: 600 ms vs 17 ms) */
  int32_t validate;       /* 1: check the CSR before searching (MCE_ERR_GRAPH on failure) */
  int32_t max_workers;    /* 0: as many wavefronts as are resident; else at most this many */
  int64_t timeout_ms;     /* wall-clock limit of one run, counted from the start of the peel; 0: 120000 */
  uint32_t flags;         /* MCE_FLAG_* */
  int32_t subgraph;       /* MCE_SUBGRAPH_* (0 = auto) */
  int32_t micro_donate_min_p; /* micro kernel: donate a batch of frames only if their |P| add up to
                             at least this; 0 = 10, else >= 1 */
  int32_t micro_stack_frames; /* micro kernel: frames per wavefront stack in device memory to start
                             with; 0 = 4096, else a power of two in [64, 2^20]. A run of mce_run or
                             mce_run_roots whose stacks overflow is run again, whole, with four
                             times as many (up to 2^20, then MCE_ERR_LIMIT); mce_stats reports the
                             size the last run used. The engine keeps the grown size for its later
                             runs. mce_run_static takes what its scratch holds instead. */
} mce_config;

/* Facts about the last graph run. */
typedef struct {
  int32_t n;
  int64_t nnz;            /* directed entries = 2 |E| */
  int32_t max_degree;     /* Delta */
  int32_t degeneracy;     /* d = largest core number */
  int32_t rounds;         /* peel rounds (the order is (round, id), see mce_ordering) */
  int32_t max_p;          /* largest |P| at a first-level subtree root (<= d) */
  int32_t max_x;          /* largest |X| at a first-level subtree root (<= Delta) */
  int64_t isolated;       /* roots with degree 0, each a maximal clique of size 1 */
  int64_t roots;          /* subtrees searched: first-level (n for mce_run) or second-level (edges) */
  uint32_t graph_errors;  /* MCE_GRAPH_* bits when the last run returned MCE_ERR_GRAPH */
  int32_t subgraph;       /* MCE_SUBGRAPH_PARTIAL or _FULL: the encoding used; 0 before the search */
  int32_t level;          /* 1: first-level subtrees (roots = vertices); 2: second-level (roots = edges) */
  int32_t complete;       /* 1: the results cover every subtree; 0: the search stopped at the time
                             limit (mce_run returned MCE_ERR_TIMEOUT) and they cover the cliques
                             found before it */
  int64_t roots_started;  /* subtree roots that were handed out: all of `roots` for a complete run;
                             after a stop, those taken by then (each finished, or abandoned at the
                             stop), plus the roots that need no search */
} mce_graph_facts;

/* Counters of the last run, summed over wavefronts. */
typedef struct {
  uint32_t struct_size;      /* sizeof(mce_run_stats) */
  int32_t workers;           /* wavefronts in the largest search launch */
  int32_t launches;          /* search launches (one per bitset width and staging sub-class) */
  int32_t handover_round;    /* -1: the search took the peel's order. Else the peel was split at
                                this round (its tail ran as a launch of its own, beside the
                                search), and the search took the hand-over order: the vertices
                                gone before the round by their rounds, then the vertices still
                                present by their degree among themselves, then id (every maximal
                                clique is reported once under any vertex order) */
  uint64_t nodes;            /* search-tree nodes whose pivot was evaluated */
  uint64_t leaves;           /* maximal cliques reported (== count minus isolated) */
  uint64_t donations;        /* branches handed to idle wavefronts (section 3.3, Table 2) */
  uint64_t pivot_rows;       /* rows scored for the pivot (P u X_P, and X_X with the full subgraph) */
  uint64_t pivot_words;      /* pivot_rows times the bitset width in 64-bit words */
  uint64_t xx_tests;         /* X_X entries tested for adjacency to a branch vertex */
  uint64_t table_words;      /* 64-bit words of induced-subgraph tables built */
  uint64_t busy_ticks;       /* sum over wavefronts of wall-clock ticks spent searching */
  uint64_t max_busy_ticks;   /* largest per-wavefront busy time */
  uint64_t max_nodes;        /* largest per-wavefront node count (section 4.3 load) */
  uint64_t kernel_ticks;     /* wall-clock ticks of the longest search launch */
  double tick_hz;            /* rate of the tick counters */
  double ms_total;           /* mce_run wall time on the host, end to end */
  double ms_validate, ms_peel, ms_orient;   /* GPU phase times, with MCE_FLAG_PHASE_TIMES */
  double ms_search;          /* search kernels alone (events around each launch), same flag or
                                MCE_FLAG_SEARCH_TIMES */
  double ms_build;           /* induced-subgraph build kernels, same flag */
  uint64_t donate_ticks;     /* sum over wavefronts of ticks spent handing branches over */
  uint64_t setup_ticks;      /* sum over wavefronts of ticks from a wake-up to the search start */
  uint64_t first_ticks;      /* sum over wavefronts of ticks from kernel start to their first task */
  uint64_t start_spread_ticks; /* largest gap between the first and last wavefront start of a launch */
  uint64_t claim_checks;     /* worker-list claim attempts by donors */
  uint64_t donate_ok_ticks;  /* ticks of the successful donations alone */
  uint64_t branches;         /* branches taken (child nodes and leaf tests); with MCE_FLAG_COUNTERS
                                for the width-1 kernel */
  uint64_t max_stack_frames; /* micro kernel: most frames one wavefront's stack held */
  int32_t micro_roots;       /* first-level subtrees searched by the micro kernel */
  int32_t micro_stack_cap;   /* frames per wavefront of the micro kernel's stack in device memory
                                (mce_config.micro_stack_frames, grown after an overflow;
                                mce_run_static: what its scratch had room for, >= 256) */
  uint64_t steps;            /* micro kernel: wavefront steps (each lane holding a frame takes one
                                node or branch) */
  uint64_t lane_steps;       /* micro kernel: lanes holding a frame, summed over steps */
  uint64_t peel_ticks[4];    /* k-core peel, as seen by its first block: barrier waits, level
                                passes, round work, total */
  int32_t launch_sub[16];    /* per search launch (up to `launches`): its sub-class (bitset width
                                class * 2 + HBM staging, or 12 for the micro kernel) */
  int32_t launch_roots[16];  /* subtrees of the launch */
  float launch_build_ms[16]; /* its induced-subgraph build, with MCE_FLAG_PHASE_TIMES */
  float launch_search_ms[16];/* its search, with MCE_FLAG_PHASE_TIMES or MCE_FLAG_SEARCH_TIMES */
  uint64_t launch_words[16]; /* per search launch: 64-bit words of the induced-subgraph tables its
                                build wrote */
  uint64_t act_cycles[7];    /* with MCE_FLAG_COUNTERS: search-kernel shader-clock cycles summed over
                                wavefronts, by activity (section 4.5 and Figure 5 break execution
                                time down the same way): [0] worker-list operations (taking subtrees,
                                answering requests, handing branches over), [1] idle (no task: asking
                                busy wavefronts for branches until one arrives or the launch ends),
                                [2] a task's start (its induced subgraph and mailbox read), [3] pivot
                                selection, [4] the branches' set operations (P n N(v), X n N(v), the
                                X_X filter, leaf tests), [5] the DFS stack (pushes, pops, spills),
                                [6] found cliques (hash, histogram). Each wavefront's seven add up to
                                its whole run; zero without the flag. The build kernels are timed by
                                launch_build_ms. */
} mce_run_stats;

/* Fills cfg with the defaults: device -1, worker_list 1, donate_min_p 1, micro_donate_min_p 10,
   validate 1, max_workers 0, timeout_ms 120000, flags 0, subgraph auto. */
mce_status mce_config_init(mce_config* cfg);

/* Creates an engine on cfg->device (cfg may be NULL for the defaults). The engine
   owns all device scratch memory; it grows on demand and is freed by mce_destroy.
   It also creates MCE_SIDE_STREAMS non-blocking streams of default priority
   (the overlapped search launches), destroyed by mce_destroy.
   On success *out receives the engine. MCE_ERR_ARG for a field out of range or a
   flag outside MCE_FLAG_*. */
mce_status mce_create(const mce_config* cfg, mce_engine** out);

/* Enumerates all maximal cliques of the graph (n vertices, nnz = row_ptr[n]
   directed entries) given as CSR in DEVICE memory: row_ptr int32[n+1],
   col_idx int32[nnz], every row sorted strictly ascending, both directions of
   each edge present. The caller owns both arrays; they must stay valid and
   unchanged until the call returns. Work is queued on `stream` (a hipStream_t;
   NULL = the null stream; the search launches fork onto the engine's own
   streams and join back, see MCE_FLAG_SERIAL) and the call returns after it
   completes. n == 0 is
   valid (count 0). nnz must be < 2^31. Results are read with mce_result. */
mce_status mce_run(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr,
                   const int32_t* col_idx, void* stream);

/* Like mce_run, but only searches the first-level subtrees of the given roots
   (section 2.4, Algorithm 3): the result covers exactly the maximal cliques
   whose earliest vertex in the degeneracy order (see mce_ordering) is one of
   roots[0..nroots). roots is an int32 array in DEVICE memory; ids must be
   distinct and in [0, n) (duplicates are counted twice). */
mce_status mce_run_roots(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr,
                         const int32_t* col_idx, const int32_t* roots, int32_t nroots,
                         void* stream);

/* Size of the static scratch array of mce_run_static, per device. */
#define MCE_STATIC_SCRATCH_BYTES (64u << 20)

/* mce_run for callers that cannot allocate (code under HIP graph capture, tight
   serving loops, harnesses that forbid hipMalloc): the same work and results,
   but every device buffer of the run (control block, peel lists, root lists,
   induced-subgraph tables, worker list, wavefront slots and frame stacks,
   counters) is carved out of one array of MCE_STATIC_SCRATCH_BYTES that the
   library holds per device in static device memory until the process ends, and
   the result read-back goes to memory inside the engine. It calls no hipMalloc,
   hipFree, hipHostMalloc or other allocating routine. The caller still owns the
   inputs (as for mce_run). Differences from mce_run: second-level runs build no
   hub adjacency bitmaps (speed only), and the micro kernel's frame stacks get
   the largest power of two up to 4096 frames per wavefront that the space left
   holds (mce_run_stats.micro_stack_cap). A graph whose buffers do not fit
   returns MCE_ERR_LIMIT with the bytes it needs in mce_last_error, before any
   search; so does a micro stack overflow during the search.
   Every call on one device shares that device's array and finds it as the
   last call left it (the run clears what must start at zero). Calls in this
   process are serialised by a lock; calls that overlap on one device from
   different processes each use their own process's array. mce_ordering and the
   per-wave counters of mce_stats / mce_worker_trace read the array, so they
   describe the last mce_run_static call on the device. The device's array
   address is looked up by mce_create (MCE_ERR_STATE if that did not happen). */
mce_status mce_run_static(mce_engine* e, int32_t n, int64_t nnz, const int32_t* row_ptr,
                          const int32_t* col_idx, void* stream);

/* Results of the last run, on the host. hist (nullable) receives
   hist[0..hist_len); hist_len = largest clique size + 1, or 0 if count == 0.
   If hist is non-NULL and hist_cap < hist_len the call returns MCE_ERR_ARG and
   still sets *hist_len. count, hash and hist_len may be NULL. After a run whose
   search stopped at the time limit the outputs are filled with the partial sums
   (the maximal cliques found before the stop; each is a maximal clique of the
   graph, but some are missing) and the call returns MCE_ERR_TIMEOUT.
   MCE_ERR_STATE if the last run produced no results (an error before the
   search, or no run yet). */
mce_status mce_result(const mce_engine* e, uint64_t* count, uint64_t* hash, uint64_t* hist,
                      int32_t hist_cap, int32_t* hist_len);

/* Graph facts of the last run (also filled when it returned MCE_ERR_GRAPH). */
mce_status mce_graph_info(const mce_engine* e, mce_graph_facts* info);

/* Copies the degeneracy order of the last run into caller DEVICE buffers of n
   int32 each: core[v] = core number of v, round[v] = the peel round that removed
   v. At level k the peel removes, in one round, every remaining vertex with at
   most k remaining neighbours; k rises to the smallest remaining degree when a
   round finds none (section 2.4 asks only for some degeneracy order; this is the
   one the engine uses). u comes after v iff (round[u], u) > (round[v], v).
   Either pointer may be NULL. Synchronous on `stream`. */
mce_status mce_ordering(const mce_engine* e, int32_t* core, int32_t* round, void* stream);

/* The bit-encoded induced subgraph (section 3.4) that the last run built for
   first-level root `root`, copied into `words` (HOST memory, cap u64 words);
   *len = its size in words, *form = its encoding: bits 0-7 the row width W in
   64-bit words, bit 8 set for a micro table (|P|, |X| <= 64: X columns follow
   the rows), bit 9 set when it holds rows for X members too (full subgraph).
   Layout, in u64 words: [0] |P| | |X| << 32; [1] root | |R| << 32 (|R| = 1);
   [2] the root's hash term (mix64(root + 0x9E3779B97F4A7C15)); then one row of
   W words per member of P, then (full) of X, members in id order within each:
   bit b of a row set iff that member is adjacent to the b-th member of P; then
   (micro) for each P member the bitset of its X neighbours (bit a: the a-th X
   member); then the P members' hash terms; then the ids of P, then of X, as
   int32, two a word (the high half of the last word is padding when
   |P| + |X| is odd). For checking the build against an independent encoding.
   MCE_ERR_STATE: no such table, because the root has no later neighbour, or
   the last run was not a complete first-level run of mce_run / mce_run_roots
   with overlapped launches (launches in series, and mce_run_static, share one
   table area that later launches overwrite). MCE_ERR_ARG: cap < *len (*len and
   *form still set). Synchronous on `stream`. */
mce_status mce_root_table(const mce_engine* e, int32_t root, uint64_t* words, int64_t cap, int64_t* len,
                          int32_t* form, void* stream);

/* Counters of the last run. stats->struct_size must be set by the caller. */
mce_status mce_stats(const mce_engine* e, mce_run_stats* stats);

/* One wavefront of a search launch in the last run (load-balance trace, section
   4.3 measures the same imbalance as nodes per SM). Ticks are the device wall
   clock (mce_run_stats.tick_hz). */
typedef struct {
  int32_t launch;           /* search launch index within the run */
  int32_t worker;           /* wavefront index within the launch */
  uint64_t start_tick;      /* the wavefront started */
  uint64_t first_tick;      /* its first task (a subtree or received branches) started; 0: none */
  uint64_t last_tick;       /* its last task ended */
  uint64_t end_tick;        /* it left the launch */
  uint64_t busy_ticks;      /* ticks holding a task */
  uint64_t nodes;           /* search-tree nodes it expanded */
  uint64_t donations;       /* branch batches it handed over */
  uint64_t received;        /* branch batches it received */
  uint64_t hw_location;     /* where it ran: XCC_ID << 32 | HW_ID as the hardware registers read
                               (HW_ID bits 11:8 compute unit, bit 12 shader array, 15:13 shader
                               engine); (XCC_ID, HW_ID bits 15:8) names one compute unit, the
                               unit of section 4.3's per-SM load */
  uint64_t leaves;          /* maximal cliques it found */
  uint64_t pivot_words;     /* with MCE_FLAG_COUNTERS: 64-bit words ANDed and counted for pivots */
  uint64_t branches;        /* with MCE_FLAG_COUNTERS: branches taken (mce_run_stats.branches) */
  uint64_t xx_tests;        /* with MCE_FLAG_COUNTERS: X_X entries tested */
} mce_worker_record;

/* Copies up to cap records of the last run's wavefronts into out (host memory)
   and stores the number available in *count. out may be NULL to query the count. */
mce_status mce_worker_trace(const mce_engine* e, mce_worker_record* out, int32_t cap, int32_t* count);

/* Text of the last error of this engine ("" if none). Valid until the next call. */
const char* mce_last_error(const mce_engine* e);

/* Name of a status code. */
const char* mce_status_string(mce_status s);

/* Frees the engine and all its device memory. NULL is ignored. */
void mce_destroy(mce_engine* e);

#ifdef __cplusplus
}
#endif

#endif /* MCE_H */
