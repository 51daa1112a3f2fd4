// Worker list shared by the search kernels ("Parallelizing Maximal Clique
// Enumeration on GPUs", section 3.3): the first-level subtree counter, the
// active count that decides termination, and branch requests between waves.
#pragma once

#include "mce_device.h"

// ------------------------------------------------------------------ worker list
// Every word two waves exchange is an agent-scope relaxed atomic; there is no
// agent-scope fence anywhere (each would write back or invalidate an L2, which
// serialises across the chip). Data is published as "atomic stores, wait for
// completion, flag store" and read after the flag with atomic loads.
#define WL_SPIN_LIMIT (1u << 22)

__device__ __forceinline__ u32* wl_flag(MceWl* wl, int w) { return &wl->line[(size_t)w * MCE_LINE_WORDS]; }
// Request slot k of wave w (the wavefront kernels use slot 0 only; the micro
// kernel takes up to MCE_REQ_SLOTS requests per step).
__device__ __forceinline__ u32* wl_req(MceWl* wl, int w, int k = 0) {
  return &wl->line[(size_t)w * MCE_LINE_WORDS + MCE_REQ_WORD + k];
}
__device__ __forceinline__ u64* wl_mask_word(MceWl* wl, int w) { return &wl->open_mask[(size_t)(w >> 6) * 16]; }
__device__ __forceinline__ u32 xorshift32(u32& x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

// A wave that starts a task accepts branch requests again. Only for a closed
// request word (before the first task, and after wl_idle): between two
// first-level subtrees the word is open and may already hold a request, which a
// plain store would erase, leaving the requester waiting for an answer.
__device__ __forceinline__ void wl_open(MceWl* wl, int wid, int nslots = 1) {
  const int lane = lane_id();
  if (lane < nslots) st_relaxed(wl_req(wl, wid, lane), 0u);
  if (lane == 0)
    __hip_atomic_fetch_or(wl_mask_word(wl, wid), 1ull << (wid & 63), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wave whose request word the open-mask shows open, drawn from one mask word
// picked at random (not this wave); -1 if that word shows none. One load per
// draw: thousands of idle waves spread their reads over all mask lines instead
// of all reading the same few. Lane 0 only.
__device__ __forceinline__ int wl_pick_open(MceWl* wl, int wid, int nworkers, u32& rng) {
  const int nwords = (nworkers + 63) >> 6;
  const int word = (int)(xorshift32(rng) % (u32)nwords);
  u64 m = ld_relaxed64(&wl->open_mask[(size_t)word * 16]);
  if (word == (wid >> 6)) m &= ~(1ull << (wid & 63));
  if (m == 0ull) return -1;
  u32 j = xorshift32(rng) % (u32)__popcll(m);
  while (j--) m &= m - 1ull;
  return word * 64 + __builtin_ctzll(m);
}

// The request word of this wave, read by every lane (uniform).
__device__ __forceinline__ u32 wl_poll(MceWl* wl, int wid) { return uni(ld_relaxed(wl_req(wl, wid))); }

// Answer a request without a branch; reopen the request slot.
__device__ __forceinline__ void wl_refuse(MceWl* wl, int wid, int rcv, int slot = 0) {
  if (lane_id() == 0) {
    st_relaxed(wl_flag(wl, rcv), MCE_FLAG_RETRY);
    st_relaxed(wl_req(wl, wid, slot), 0u);
  }
}

// Hand a branch to rcv after its mailbox was written with atomic stores: count
// it active (before this wave can ever give up its own share: same-address
// atomics of one wave stay in order, and the wait below completes the
// increment before the receiver can run), wake it, reopen the request word.
__device__ __forceinline__ void wl_give(MceWl* wl, int wid, int rcv) {
  if (lane_id() == 0) __hip_atomic_fetch_add(&wl->n_active, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_stores_complete();
  if (lane_id() == 0) {
    st_relaxed(wl_flag(wl, rcv), MCE_FLAG_TASK);
    st_relaxed(wl_req(wl, wid), 0u);
  }
}

// Receiver side (section 3.3). Closes this wave's request word (refusing a
// request that raced in), gives up its share of n_active, and asks busy waves,
// drawn at random from the open-mask, for a branch until one arrives. The wave
// that brings n_active to zero (no task held anywhere; only active waves hand
// out branches, so none can appear) writes MCE_FLAG_EXIT into every wake flag.
// Returns 1 with a task in the mailbox (the donor counted this wave active
// again), 0 to exit. Whole wave; the shared words are touched by lane 0.
// Ordering: the refusal and the flag reset complete before the share is given
// up, and an answer flag is only consumed with a compare-and-swap, so the exit
// broadcast (issued after every share release) cannot be overwritten.
__device__ int wl_idle(MceWl* wl, int wid, int nworkers, u64 deadline, u32* status, u32& rng, int nslots = 1) {
  const int lane = lane_id();
  u32* my = wl_flag(wl, wid);
  int left = 0;
  if (lane < nslots) {   // close every slot, refusing a request that raced in
    const u32 old = __hip_atomic_exchange(wl_req(wl, wid, lane), MCE_REQ_CLOSED, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    if (old != 0u && old != MCE_REQ_CLOSED) st_relaxed(wl_flag(wl, (int)old - 1), MCE_FLAG_RETRY);
  }
  if (lane == 0) {
    __hip_atomic_fetch_and(wl_mask_word(wl, wid), ~(1ull << (wid & 63)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    st_relaxed(my, 0u);
  }
  wait_stores_complete();
  if (lane == 0) {
    left = __hip_atomic_fetch_add(&wl->n_active, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - 1;
    if (left < 0) atomicOr(status, MCE_E_PROTO);
  }
  left = read_lane(left, 0);
  int res = 0;
  if (left > 0 && nworkers > 1) {
    u32 fails = 0, it = 0;
    for (;;) {
      int stop = 0;
      if (lane == 0) {
        if (ld_relaxed(my) == MCE_FLAG_EXIT) {
          stop = 1;
        } else if ((++it & 15u) == 0) {
          if (ld_relaxed(&wl->done)) {
            stop = 1;   // another wave stopped the launch on an error
          } else if (past_deadline(deadline)) {
            atomicOr(status, MCE_E_TIMEOUT);
            st_relaxed(&wl->done, 1u);
            stop = 1;
          }
        }
      }
      if (read_lane(stop, 0)) break;
      int asked = 0;
      if (lane == 0) {
        const int v = wl_pick_open(wl, wid, nworkers, rng);
        const int k = nslots > 1 ? (int)(xorshift32(rng) % (u32)nslots) : 0;
        u32 expected = 0u;
        if (v >= 0 && ld_relaxed(wl_req(wl, v, k)) == 0u &&
            __hip_atomic_compare_exchange_strong(wl_req(wl, v, k), &expected, (u32)wid + 1u, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          asked = 1;
          // wait for the answer: the asked wave reads its request word once per node
          u32 spins = 0;
          for (;;) {
            const u32 a = ld_relaxed(my);
            if (a == MCE_FLAG_TASK) {
              res = 1;
              stop = 1;
              break;
            }
            if (a == MCE_FLAG_EXIT) {
              stop = 1;
              break;
            }
            if (a == MCE_FLAG_RETRY) {
              u32 e = MCE_FLAG_RETRY;
              if (!__hip_atomic_compare_exchange_strong(my, &e, 0u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT))
                stop = 1;   // the exit broadcast replaced the refusal
              break;
            }
            if ((++spins & 255u) == 0) {
              if (ld_relaxed(&wl->done)) {
                stop = 1;
                break;
              }
              if (past_deadline(deadline)) {
                atomicOr(status, MCE_E_TIMEOUT);
                st_relaxed(&wl->done, 1u);
                stop = 1;
                break;
              }
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
      }
      if (read_lane(stop, 0)) break;
      if (read_lane(asked, 0)) {
        fails = 0;
      } else {
        // nobody open, or the wave asked is busy with another request: back off
        ++fails;
        if (fails < 16) __builtin_amdgcn_s_sleep(2);
        else if (fails < 64) __builtin_amdgcn_s_sleep(8);
        else __builtin_amdgcn_s_sleep(16);
      }
    }
  }
  res = read_lane(res, 0);
  if (left <= 0) {
    for (int i = lane; i < nworkers; i += MCE_WAVE) st_relaxed(wl_flag(wl, i), MCE_FLAG_EXIT);
  }
  return res;
}

// Phase 1 (section 3.3): the next first-level subtree from the shared counter,
// or nroots when none is left. Every subtree goes through the counter: a wave
// that has not started yet must never hold a subtree that other waves count as
// taken, or they could finish and leave while it still needs the worker list.
// Roots go out in chunks: one fetch takes about the roots left divided by
// 2 x nworkers (at least 1, at most maxc), so that hundreds of thousands of tiny
// subtrees do not each cost an atomic on the one shared counter (same-address
// atomics from thousands of waves serialise), while the last roots, and the
// few roots of a launch with more waves than roots, still go out one at a time.
struct RootCursor {
  u32 next, end;   // this wave's chunk [next, end)
};
__device__ __forceinline__ u32 take_root(MceWl* wl, RootCursor& rc, u32 nroots, u32 nworkers, u32 maxc) {
  if (rc.next >= rc.end) {
    u32 idx = nroots, c = 0;
    if (lane_id() == 0) {
      const u32 seen = ld_relaxed(&wl->root_ctr);
      if (seen < nroots) {
        c = min(maxc, max(1u, (nroots - seen) / (2u * nworkers)));
        idx = atomicAdd(&wl->root_ctr, c);
      }
    }
    idx = (u32)read_lane((int)idx, 0);
    c = (u32)read_lane((int)c, 0);
    if (idx >= nroots) return nroots;
    rc.next = idx;
    rc.end = min(idx + c, nroots);
  }
  return rc.next++;
}

// Count this wave active, and wait until the increment is performed: it must
// precede the wave's first root-counter increment, or another wave could see
// the roots gone and the count at zero while this wave holds a subtree.
__device__ __forceinline__ void wl_join(MceWl* wl) {
  if (lane_id() == 0) __hip_atomic_fetch_add(&wl->n_active, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_stores_complete();
}

