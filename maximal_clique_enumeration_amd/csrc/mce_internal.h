// Internal interface between the engine (host) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mce_device.h"

struct ClassOffsets {
  int off[MCE_NCLASS];
};

// Per-wavefront statistics written by the search kernel (u64 each).
enum {
  ST_NODES = 0,
  ST_LEAVES,
  ST_DONATIONS,
  ST_PIVOT_ROWS,
  ST_PIVOT_WORDS,
  ST_XX_TESTS,
  ST_IP_ROWS,
  ST_BUSY_TICKS,
  ST_ROOTS,
  ST_RECEIVED,
  ST_TOTAL_TICKS,
  MCE_NSTAT
};

struct SearchParams {
  const int* rp;
  const int* ci;
  const int* rnd;
  const int* roots;      // this launch's first-level subtree roots
  int nroots;
  int nworkers;
  u64* g_hist;           // global histogram (MCE_MAX_P + 2 entries)
  u64* g_hash;
  MceWl* wl;
  char* slots;           // one HBM slot per wavefront
  size_t slot_bytes;
  size_t off_rows, off_hv, off_pid, off_stack, off_xx, off_mail;
  int donate_min_p;
  int worker_list;
  u64 budget;            // wall-clock ticks after which the launch is abandoned
  u32* status;
  u64* stats;            // nworkers * MCE_NSTAT
};

// Slot layout for a width class: byte offsets and total size per wavefront.
struct SlotLayout {
  size_t off_rows, off_hv, off_pid, off_stack, off_xx, off_mail, bytes;
};
SlotLayout mce_slot_layout(int wclass, int max_x);
size_t mce_search_lds_bytes(int wclass, bool lds_rows, bool lds_stack);
bool mce_search_lds_rows(int wclass);
bool mce_search_lds_stack(int wclass);

hipError_t mce_launch_validate(int n, long long nnz, const int* rp, const int* ci, MceCtl* ctl, int blocks,
                               hipStream_t s);
hipError_t mce_launch_peel(int n, const int* rp, const int* ci, int* deg, int* rnd, int* core, int* alive0,
                           int* alive1, int* front0, int* front1, MceCtl* ctl, u64 budget, int blocks,
                           hipStream_t s);
int mce_peel_max_blocks(int num_cu);
hipError_t mce_launch_orient(int n, const int* rp, const int* ci, const int* rnd, const int* roots, int nroots,
                             int* pcount, MceCtl* ctl, int blocks, hipStream_t s);
hipError_t mce_launch_bucket(int n, const int* roots, int nroots, const int* pcount, ClassOffsets off, int* lists,
                             MceCtl* ctl, int blocks, hipStream_t s);

// Resident wavefronts of the search kernel of a class over the whole chip (0 on error).
int mce_search_max_workers(int wclass, bool hbm_staging, int num_cu);
hipError_t mce_launch_search(int wclass, bool hbm_staging, const SearchParams& prm, hipStream_t s);

hipError_t mce_launch_wl_init(MceWl* wl, hipStream_t s);
