// ra_ring.cpp -- one whole lap of the ring for one rank, emulated on one GPU.
//
// The P KV blocks of the lap are resident in device memory.  Step 0 attends the rank's
// own block in place; the block for step s+1 is "received" into one of two receive
// buffers by a hipMemcpyAsync on a side stream while step s's kernel runs on the compute
// stream ("GPU ring attention", section "Hiding the ring behind the GEMMs": the transfer
// for the next block is posted on a separate stream and the kernel runs against the
// buffer it already owns).  Events carry the two hazards the double-buffer scheme must
// respect ("Ring Attention：把超长序列沿设备环流动", section 双缓冲是重叠成立的基础): a receive
// buffer is not overwritten before the kernel that reads it has finished (ev_free), and
// the kernel does not read a buffer before its transfer has landed (ev_ready).  A block that
// no query of the rank sees (a causal block wholly in the future) launches no kernel: its
// buffer is free once it has landed, and the next transfer into it waits for nothing else.
//
// Block visit order: at step s rank r holds block (r - s) mod P, the order of the
// four-device table on the same page (section 环是怎样工作的).
//
// The last step finalizes as it writes back when one launch covers all of it and every row
// sees a key (the output normalisation of "GPU ring attention", section "Why partial results
// are allowed to merge", applied in the step kernel's write-back): one pass over the state less.

#include <hip/hip_runtime.h>

#include <cstdio>

#include "../../include/ra.h"
#include "ra_internal.h"

namespace ra {
int set_error(int code, const char* msg);
int set_hip_error(hipError_t e, const char* what);
int block_step_final(ra_state* st, const void* k, const void* v, int32_t kv_len, int32_t mask_kind,
                     int64_t q_offset, int64_t k_offset, float* o, float* lse, int* finalized);
}  // namespace ra

namespace {

struct Events {
  hipEvent_t start = nullptr, ready[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr};
  ~Events() {
    if (start) (void)hipEventDestroy(start);
    for (int i = 0; i < 2; ++i) {
      if (ready[i]) (void)hipEventDestroy(ready[i]);
      if (freed[i]) (void)hipEventDestroy(freed[i]);
    }
  }
};

struct StateGuard {
  ra_state* st = nullptr;
  ~StateGuard() {
    if (st) ra_state_destroy(st);
  }
};

}  // namespace

extern "C" int ra_ring_lap_emulated(const ra_desc* desc, const void* q, void* workspace,
                                    const ra_lap* lap, float* o, float* lse, ra_stats* stats_out) {
  if (!desc || !lap) return ra::set_error(RA_E_INVALID, "desc or lap is NULL");
  const int P = desc->ring_size;
  if (P < 1) return ra::set_error(RA_E_INVALID, "ring_size must be >= 1");
  if (lap->rank < 0 || lap->rank >= P) return ra::set_error(RA_E_INVALID, "rank out of range");
  if (!lap->k_blocks || !lap->v_blocks) return ra::set_error(RA_E_INVALID, "block arrays are NULL");
  if (lap->kv_len < 0) return ra::set_error(RA_E_INVALID, "kv_len must be >= 0");
  if (P > 1 && lap->kv_len > 0) {
    for (int i = 0; i < 2; ++i)
      if (!lap->recv_k[i] || !lap->recv_v[i])
        return ra::set_error(RA_E_INVALID, "receive buffers are NULL");
    if (lap->block_bytes == 0) return ra::set_error(RA_E_INVALID, "block_bytes is 0");
  }
  for (int j = 0; j < P; ++j) {
    if (lap->kv_len > 0 && (!lap->k_blocks[j] || !lap->v_blocks[j]))
      return ra::set_error(RA_E_INVALID, "a KV block pointer is NULL");
    if (lap->kv_valid && (lap->kv_valid[j] < 0 || lap->kv_valid[j] > lap->kv_len)) {
      char msg[96];
      snprintf(msg, sizeof msg, "kv_valid[%d] = %d is outside [0, kv_len]", j, (int)lap->kv_valid[j]);
      return ra::set_error(RA_E_INVALID, msg);
    }
  }

  StateGuard g;
  int rc = ra_state_init(desc, q, workspace, &g.st);
  if (rc) return rc;

  hipStream_t cs = static_cast<hipStream_t>(desc->stream);
  hipStream_t ss = static_cast<hipStream_t>(lap->side_stream);
  Events ev;
  hipError_t e = hipEventCreateWithFlags(&ev.start, hipEventDisableTiming);
  for (int i = 0; i < 2 && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&ev.ready[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev.freed[i], hipEventDisableTiming);
  }
  if (e != hipSuccess) return ra::set_hip_error(e, "event create");
  // the side stream starts after everything already queued on the compute stream
  if ((e = hipEventRecord(ev.start, cs)) != hipSuccess) return ra::set_hip_error(e, "event record");
  if ((e = hipStreamWaitEvent(ss, ev.start, 0)) != hipSuccess) return ra::set_hip_error(e, "stream wait");

  const int r = lap->rank;
  const bool copies = lap->kv_len > 0 && P > 1;
  int finalized = 0;
  // positions of step s's block, and whether any query of this rank sees a key of it
  auto offsets = [&](int j, int64_t* q_off, int64_t* k_off) {
    *q_off = 0;
    *k_off = 0;
    if (lap->mask_kind == RA_MASK_CAUSAL_CONTIGUOUS) {
      *q_off = (int64_t)r * desc->q_len;
      *k_off = (int64_t)j * lap->kv_len;
    } else if (lap->mask_kind == RA_MASK_CAUSAL_STRIPED || lap->mask_kind == RA_MASK_CAUSAL_ZIGZAG) {
      *q_off = r;
      *k_off = j;
    }
  };
  auto keys_of = [&](int j) { return lap->kv_valid ? lap->kv_valid[j] : lap->kv_len; };
  auto runs = [&](int s) {
    const int j = ((r - s) % P + P) % P;
    int64_t qo, ko;
    offsets(j, &qo, &ko);
    ra_stats st;
    return ra_plan_block(desc, keys_of(j), lap->mask_kind, qo, ko, &st) != RA_OK || st.blocks_run > 0;
  };
  for (int s = 0; s < P; ++s) {
    const int j = ((r - s) % P + P) % P;
    if (copies && s + 1 < P) {  // post the receive of the next block
      const int nb = (s + 1) & 1;
      const int jn = ((r - s - 1) % P + P) % P;
      // the buffer's previous block (step s - 1) must have been read by its kernel; a block
      // that no query sees launches nothing and frees its buffer as soon as it has landed,
      // which the side stream's own order already gives
      if (s + 1 >= 3 && runs(s - 1) && (e = hipStreamWaitEvent(ss, ev.freed[nb], 0)) != hipSuccess)
        return ra::set_hip_error(e, "stream wait");
      if (lap->poison) {
        if ((e = hipMemsetAsync(lap->recv_k[nb], 0xFF, lap->block_bytes, ss)) != hipSuccess ||
            (e = hipMemsetAsync(lap->recv_v[nb], 0xFF, lap->block_bytes, ss)) != hipSuccess)
          return ra::set_hip_error(e, "poison fill");
      }
      if ((e = hipMemcpyAsync(lap->recv_k[nb], lap->k_blocks[jn], lap->block_bytes,
                              hipMemcpyDeviceToDevice, ss)) != hipSuccess ||
          (e = hipMemcpyAsync(lap->recv_v[nb], lap->v_blocks[jn], lap->block_bytes,
                              hipMemcpyDeviceToDevice, ss)) != hipSuccess)
        return ra::set_hip_error(e, "block copy");
      if ((e = hipEventRecord(ev.ready[nb], ss)) != hipSuccess) return ra::set_hip_error(e, "event record");
    }
    const void* kp = lap->k_blocks[j];
    const void* vp = lap->v_blocks[j];
    if (copies && s > 0) {
      if ((e = hipStreamWaitEvent(cs, ev.ready[s & 1], 0)) != hipSuccess)
        return ra::set_hip_error(e, "stream wait");
      kp = lap->recv_k[s & 1];
      vp = lap->recv_v[s & 1];
    }
    int64_t q_off, k_off;
    offsets(j, &q_off, &k_off);
    if (lap->step_events &&
        (e = hipEventRecord(static_cast<hipEvent_t>(lap->step_events[2 * s]), cs)) != hipSuccess)
      return ra::set_hip_error(e, "event record");
    // padding past a block's real keys is cut off by the key count: no query sees it
    const int32_t keys = keys_of(j);
    // the last block may finalize as its launch writes back (then no separate finalize pass)
    rc = s + 1 < P ? ra_block_step(g.st, kp, vp, keys, lap->mask_kind, q_off, k_off)
                   : ra::block_step_final(g.st, kp, vp, keys, lap->mask_kind, q_off, k_off, o, lse, &finalized);
    if (rc) return rc;
    if (lap->step_events &&
        (e = hipEventRecord(static_cast<hipEvent_t>(lap->step_events[2 * s + 1]), cs)) != hipSuccess)
      return ra::set_hip_error(e, "event record");
    if (copies && s > 0 && (e = hipEventRecord(ev.freed[s & 1], cs)) != hipSuccess)
      return ra::set_hip_error(e, "event record");
  }
  if (!finalized && (rc = ra_finalize(g.st, o, lse)) != RA_OK) return rc;
  if (stats_out) ra_get_stats(g.st, stats_out);
  return RA_OK;
}
