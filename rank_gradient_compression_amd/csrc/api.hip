// C ABI entry points that touch the device: workspace set-up, the PowerSGD
// compression step, decompression, refresh, timing and the copy kernel.
//
// The step follows the "Method" section of the anthology note on PowerSGD
// (note 152): P = M Q, all-reduce P, orthogonalise, Q = M^T P_hat, all-reduce
// Q; the all-reduces are the caller's aggregation hook.  Every call only
// enqueues work on the caller's stream: no host synchronisation and no
// device allocation.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "psgd_internal.h"
#include "psgd_kernels.h"
#include "psgd_flat.h"
#include "psgd_payload.h"

namespace psgd {

// -------------------------------------------------------------------- timing

struct TimingRecord {
  int stage;
  hipEvent_t start, stop;
};

struct TimingState {
  bool enabled = false;
  bool reserved = false;  // the up-front event pool has been created
  uint32_t mask = ~0u;    // stages that record events (bit s = stage s)
  std::vector<TimingRecord> records;
  std::vector<hipEvent_t> pool;
};

static hipEvent_t take_event(TimingState* t) {
  if (!t->pool.empty()) {
    hipEvent_t e = t->pool.back();
    t->pool.pop_back();
    return e;
  }
  // Timing-only events: no system-scope fence (cache writeback and
  // invalidation) when recorded, so that timing does not perturb the stages.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Records events around one stage when timing is enabled.
class StageTimer {
 public:
  StageTimer(psgd_plan* p, int stage, hipStream_t s) : p_(p), stage_(stage), s_(s) {
    if (!p_->timing || !p_->timing->enabled || !((p_->timing->mask >> stage_) & 1u)) return;
    std::lock_guard<std::mutex> lk(p_->timing_mu);
    start_ = take_event(p_->timing);
    stop_ = take_event(p_->timing);
    if (start_ && stop_) (void)hipEventRecord(start_, s_);
  }
  ~StageTimer() {
    if (!start_ || !stop_) return;
    (void)hipEventRecord(stop_, s_);
    std::lock_guard<std::mutex> lk(p_->timing_mu);
    p_->timing->records.push_back({stage_, start_, stop_});
  }

 private:
  psgd_plan* p_;
  int stage_;
  hipStream_t s_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

// ------------------------------------------------------------------ helpers

// Buffers are accessed with 16-byte vector instructions from their base.
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static LaunchCtx make_ctx(const psgd_plan* p, void* ws, hipStream_t s) {
  const WsHeader& h = p->hdr;
  char* b = static_cast<char*>(ws);
  LaunchCtx c{};
  c.stream = s;
  c.rank = p->rank;
  c.rank_pad = h.rank_pad;
  c.mfma = h.mfma != 0;
  c.g_bf16 = (p->flags & PSGD_FLAG_GRADS_BF16) != 0;
  c.stream_hint = (int64_t)p->dense * 4 > kStreamHintBytes;
  c.nmat = h.nmat;
  c.npass = h.npass;
  c.wg_rows = h.wg_rows;
  c.wg_rows_v4 = h.wg_rows_v4;
  c.wg_rec = h.wg_rec;
  c.wg_mtp = h.wg_mtp;
  c.wg_red = h.wg_red;
  c.wg_pass = h.wg_pass;
  c.wg_pred = h.wg_pred;
  c.wg_gram = h.wg_gram;
  c.wg_gramq = h.wg_gramq;
  c.mats = reinterpret_cast<const MatDesc*>(b + h.mat_off);
  c.pass = reinterpret_cast<const PassDesc*>(b + h.pass_off);
  c.orth = reinterpret_cast<const OrthDesc*>(b + h.orth_off);
  c.rows_map = reinterpret_cast<const int32_t*>(b + h.rows_map_off);
  c.rec_map = reinterpret_cast<const int32_t*>(b + h.rec_map_off);
  c.mtp_map = reinterpret_cast<const int32_t*>(b + h.mtp_map_off);
  c.red_map = reinterpret_cast<const int32_t*>(b + h.red_map_off);
  c.pass_map = reinterpret_cast<const int32_t*>(b + h.pass_map_off);
  c.pred_map = reinterpret_cast<const int32_t*>(b + h.pred_map_off);
  c.gram_map = reinterpret_cast<const int32_t*>(b + h.gram_map_off);
  c.gramq_map = reinterpret_cast<const int32_t*>(b + h.gramq_map_off);
  c.part = reinterpret_cast<float*>(b + h.part_base);
  c.ppart = b + h.ppart_base;
  c.gram = reinterpret_cast<double*>(b + h.gram_base);
  c.rscr = reinterpret_cast<float*>(b + h.refresh_base);
  return c;
}

// Workgroups of matrix k in one of the plan's grids.
static GridRange mat_range(const psgd_plan* p, size_t k, int32_t MatDesc::*first, int total) {
  const int b = p->mats[k].*first;
  const int e = k + 1 < p->mats.size() ? p->mats[k + 1].*first : total;
  return GridRange{b, e - b};
}

// ---- the stages of one step, dispatched to the vector or matrix-core kernels

// P = M Q for the grid range g (mode as in launch_ef_p), into P at the plan's
// offsets (p_fixed < 0) or at p_fixed, column-split partials summed.
static hipError_t stage_mq(const psgd_plan* p, const LaunchCtx& c, const GridRange& g, const GridRange& gp, int mode,
                           const void* G, float* E, float* U, const float* Q, float* P, int64_t p_fixed) {
  hipError_t e = c.mfma ? launch_mfma_p(c, g, mode, G, E, U, p->beta, Q, P, p_fixed)
                        : launch_ef_p(c, g, mode, G, E, U, p->beta, Q, P, p_fixed);
  if (e != hipSuccess) return e;
  return launch_psum(c, gp, P, p_fixed);
}

// Orthonormalise the P factors of all matrices (P in `base` at the plan's
// offsets).
static hipError_t stage_orth_all_p(const LaunchCtx& c, float* base, int32_t* zcount = nullptr) {
  return launch_gram_orth(c, 0, c.nmat, c.gram_map, c.wg_gram, base, zcount);
}

// Orthonormalise the Q factors of all matrices (the refresh).
static hipError_t stage_orth_all_q(const LaunchCtx& c, float* q) {
  return launch_gram_orth(c, 2 * c.nmat, c.nmat, c.gramq_map, c.wg_gramq, q);
}

// Q = M^T P_hat (row-block partials reduced in fixed order).
static hipError_t stage_mtp(const LaunchCtx& c, const GridRange& g, const GridRange& gr, const float* M,
                            const float* Ph, int64_t ph_fixed, float* Q) {
  hipError_t e = c.mfma ? launch_mfma_qt(c, g, M, Ph, ph_fixed, Q) : launch_mtp(c, g, M, Ph, ph_fixed, Q);
  if (e != hipSuccess) return e;
  return launch_qreduce(c, gr, Q);
}

// (flat_lds: the plan's dynamic LDS for flat-tiled matrices on the vector path)
static hipError_t stage_recon(const psgd_plan* p, const LaunchCtx& c, float* E, const float* Q, const float* Ph,
                              float* Mhat, bool residual, const SgdArgs& sg) {
  return c.mfma ? launch_mfma_recon(c, E, Q, Ph, Mhat, residual, sg)
                : launch_recon_lds(c, E, Q, Ph, Mhat, residual, sg, p->flat_lds);
}

static psgd_status_t check_ws(const psgd_plan* p, const void* ws, size_t bytes, const char* fn) {
  if (!ws) {
    set_error("%s: workspace is NULL", fn);
    return PSGD_ERR_WORKSPACE;
  }
  if (((uintptr_t)ws & 255u) != 0) {
    set_error("%s: workspace is not 256-byte aligned", fn);
    return PSGD_ERR_WORKSPACE;
  }
  if (bytes < (size_t)p->hdr.total_bytes) {
    set_error("%s: workspace of %zu bytes, the plan needs %lld", fn, bytes, (long long)p->hdr.total_bytes);
    return PSGD_ERR_WORKSPACE;
  }
  return PSGD_OK;
}

static psgd_status_t hip_fail(hipError_t e, const char* what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return PSGD_ERR_HIP;
}

#define PSGD_LAUNCH(stage, expr, what)                   \
  do {                                                   \
    StageTimer _t(p, stage, stream);                     \
    const hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return hip_fail(_e, what);     \
  } while (0)

}  // namespace psgd

using namespace psgd;

extern "C" void psgd_plan_destroy(psgd_plan_t p) {
  if (!p) return;
  if (p->timing) {
    for (auto& r : p->timing->records) {
      (void)hipEventDestroy(r.start);
      (void)hipEventDestroy(r.stop);
    }
    for (hipEvent_t e : p->timing->pool) (void)hipEventDestroy(e);
    delete p->timing;
  }
  delete p;
}

extern "C" psgd_status_t psgd_workspace_init(psgd_plan_t p, void* ws, size_t bytes, hipStream_t stream) {
  clear_error();
  if (!p) {
    set_error("psgd_workspace_init: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (psgd_status_t s = check_ws(p, ws, bytes, "psgd_workspace_init")) return s;
  if (p->tables.empty()) return PSGD_OK;
  const hipError_t e = hipMemcpyAsync(ws, p->tables.data(), p->tables.size(), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "psgd_workspace_init: table upload");
  return PSGD_OK;
}

// Argument checks of psgd_compress and psgd_compress_noalloc (host only; no
// device call).  On success *o holds the step options.
static psgd_status_t validate_compress(const char* fn, const psgd_plan* p, const void* grads, const float* err,
                                       const float* mom, const float* q, const float* pbuf, const float* mhat,
                                       const psgd_step_opts_t* opts, psgd_step_opts_t* o) {
  if (!p) {
    set_error("%s: plan is NULL", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  const bool momentum = (p->flags & PSGD_FLAG_MOMENTUM) != 0;
  const bool any = p->ntensors > 0;
  if (any && (!grads || !pbuf || (!p->mats.empty() && (!err || !q)))) {
    set_error("%s: a required buffer is NULL", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if (momentum && any && !mom) {
    set_error("%s: the plan compresses momentum but mom is NULL", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if (!momentum && mom) {
    set_error("%s: mom given but the plan has no momentum flag", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if (!aligned16(grads) || !aligned16(err) || !aligned16(mom) || !aligned16(q) || !aligned16(pbuf) ||
      !aligned16(mhat)) {
    set_error("%s: buffers must be 16-byte aligned", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if (mhat && (mhat == err || mhat == mom)) {
    set_error("%s: mhat may alias grads only", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if (mhat && (p->flags & PSGD_FLAG_GRADS_BF16) && (const void*)mhat == grads) {
    set_error("%s: mhat (fp32) cannot alias bfloat16 gradients", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  *o = psgd_step_opts_t{};
  if (opts) *o = *opts;
  if (o->power_iters < 0 || o->refresh_iters < 0) {
    set_error("%s: negative iteration count", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  constexpr uint32_t kKnownStepFlags =
      PSGD_STEP_NO_ERROR_FEEDBACK | PSGD_STEP_NESTEROV | PSGD_STEP_DEFER_RESIDUAL | PSGD_STEP_RESIDUAL_DEFERRED |
      PSGD_STEP_PAYLOAD_BF16 | PSGD_STEP_PAYLOAD_FP8;
  if (o->flags & ~kKnownStepFlags) {
    set_error("%s: unknown step flag bits 0x%x", fn, o->flags & ~kKnownStepFlags);
    return PSGD_ERR_INVALID_ARG;
  }
  if ((o->flags & PSGD_STEP_PAYLOAD_BF16) && (o->flags & PSGD_STEP_PAYLOAD_FP8)) {
    set_error("%s: PSGD_STEP_PAYLOAD_BF16 and PSGD_STEP_PAYLOAD_FP8 are exclusive", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if ((o->flags & (PSGD_STEP_DEFER_RESIDUAL | PSGD_STEP_RESIDUAL_DEFERRED)) &&
      (o->flags & PSGD_STEP_NO_ERROR_FEEDBACK)) {
    set_error("%s: a deferred residual needs error feedback", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if ((o->params != nullptr) != (o->sgd_buf != nullptr) || !aligned16(o->params) || !aligned16(o->sgd_buf)) {
    set_error("%s: params and sgd_buf must be given together, 16-byte aligned", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if (((uintptr_t)o->zero_cols & 3u) != 0) {
    set_error("%s: zero_cols must be 4-byte aligned", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  if (o->params && (o->params == err || o->params == mom || o->params == mhat || o->sgd_buf == err ||
                    o->sgd_buf == mom || o->sgd_buf == mhat || o->params == o->sgd_buf)) {
    set_error("%s: params / sgd_buf must not alias the other buffers", fn);
    return PSGD_ERR_INVALID_ARG;
  }
  return PSGD_OK;
}

// The step itself, on validated arguments and an initialised workspace `ws`
// (the caller's, or the library's static scratch).
static psgd_status_t run_compress(psgd_plan* p, const void* grads, float* err, float* mom, float* q, float* pbuf,
                                  float* mhat, const psgd_step_opts_t& o, psgd_reduce_fn hook, void* user, void* ws,
                                  hipStream_t stream) {
  const bool momentum = (p->flags & PSGD_FLAG_MOMENTUM) != 0;
  const bool defer_out = (o.flags & PSGD_STEP_DEFER_RESIDUAL) != 0;
  const bool defer_in = (o.flags & PSGD_STEP_RESIDUAL_DEFERRED) != 0;
  const int refresh_iters = o.refresh_iters;
  const int power_iters = o.power_iters > 1 ? o.power_iters : 1;
  const bool ef = (o.flags & PSGD_STEP_NO_ERROR_FEEDBACK) == 0;
  const bool payload_bf16 = (o.flags & PSGD_STEP_PAYLOAD_BF16) != 0;
  const bool payload_fp8 = (o.flags & PSGD_STEP_PAYLOAD_FP8) != 0;
  const SgdArgs sg{o.params, o.sgd_buf, o.sgd_lr, o.sgd_momentum, (o.flags & PSGD_STEP_NESTEROV) ? 1 : 0};
  if (p->ntensors == 0) return PSGD_OK;

  LaunchCtx c = make_ctx(p, ws, stream);
  c.p_prev = pbuf;
  float* U = momentum ? mom : nullptr;
  const GridRange all_rows{0, c.wg_rows}, all_pred{0, c.wg_pred}, all_mtp{0, c.wg_mtp}, all_red{0, c.wg_red};
  const int mode = !ef ? (momentum ? 4 : 3) : defer_in ? (momentum ? 6 : 5) : (momentum ? 2 : 1);

  // The pass-through values are packed into the P buffer: by the first
  // pass's extra workgroups on the vector path, by a launch of their own on
  // the matrix-core path.
  LaunchCtx c1 = c;
  if (c.mfma && c.wg_pass > 0)  // (no stage, and no timing events, without pass-through tensors)
    PSGD_LAUNCH(PSGD_STAGE_PASSTHRU, launch_pass_pack(c, grads, U, p->beta, pbuf), "pass-through pack");
  else
    c1.pack_dst = pbuf;
  if (refresh_iters <= 0) {
    PSGD_LAUNCH(PSGD_STAGE_EF_P, stage_mq(p, c1, all_rows, all_pred, mode, grads, err, U, q, pbuf, -1),
                "EF-add + P = M Q");
  } else {
    // PowerSGD+ step: M = X + E first, then the subspace refresh of every
    // warm-start Q on M, then P = M Q with the refreshed Q.
    PSGD_LAUNCH(PSGD_STAGE_EF_P, stage_mq(p, c1, all_rows, all_pred, mode, grads, err, U, q, c.rscr, -1),
                "EF-add");
    for (int it = 0; it < refresh_iters; ++it) {
      PSGD_LAUNCH(PSGD_STAGE_REFRESH, stage_mq(p, c, all_rows, all_pred, 0, nullptr, err, nullptr, q, c.rscr, -1),
                  "refresh: P = M Q");
      PSGD_LAUNCH(PSGD_STAGE_REFRESH, stage_orth_all_p(c, c.rscr), "refresh: orthonormalise P");
      PSGD_LAUNCH(PSGD_STAGE_REFRESH, stage_mtp(c, all_mtp, all_red, err, c.rscr, -1, q), "refresh: Q = M^T P");
      PSGD_LAUNCH(PSGD_STAGE_REFRESH, stage_orth_all_q(c, q), "refresh: orthonormalise Q");
    }
    PSGD_LAUNCH(PSGD_STAGE_EF_P, stage_mq(p, c, all_rows, all_pred, 0, nullptr, err, nullptr, q, pbuf, -1),
                "P = M Q");
  }
  // One (or power_iters) subspace iterations, with both aggregation hooks in
  // each; later iterations start again from P = M Q with the new Q.
  for (int it = 0; it < power_iters; ++it) {
    if (it > 0)
      PSGD_LAUNCH(PSGD_STAGE_EF_P, stage_mq(p, c, all_rows, all_pred, 0, nullptr, err, nullptr, q, pbuf, -1),
                  "P = M Q");
    if (payload_bf16)  // the factors only; pass-through values stay fp32
      PSGD_LAUNCH(PSGD_STAGE_EF_P, launch_round_bf16(pbuf, (int64_t)p->p_elems, stream), "round P to bfloat16");
    else if (payload_fp8)  // per column of each matrix's P
      PSGD_LAUNCH(PSGD_STAGE_EF_P, launch_round_fp8_cols(c, 0, pbuf), "round P to fp8");
    // The pass-through values ride with the first P only: later iterations
    // aggregate the factors alone, so those values are averaged exactly once.
    const size_t p_count = it == 0 ? p->p_elems + p->pt_elems : p->p_elems;
    if (hook && p_count > 0 && hook(pbuf, p_count, stream, user) != 0) {
      set_error("psgd_compress: aggregation hook failed on P");
      return PSGD_ERR_HOOK;
    }
    PSGD_LAUNCH(PSGD_STAGE_GS, stage_orth_all_p(c, pbuf, o.zero_cols), "orthogonalise P");
    {
      StageTimer _t(p, PSGD_STAGE_MTP, stream);
      const hipError_t e =
          c.mfma ? launch_mfma_qt(c, all_mtp, err, pbuf, -1, q) : launch_mtp(c, all_mtp, err, pbuf, -1, q);
      if (e != hipSuccess) return hip_fail(e, "Q = M^T P_hat");
    }
    PSGD_LAUNCH(PSGD_STAGE_QREDUCE, launch_qreduce(c, all_red, q), "Q partial reduction");
    if (payload_bf16)
      PSGD_LAUNCH(PSGD_STAGE_QREDUCE, launch_round_bf16(q, (int64_t)p->q_elems, stream), "round Q to bfloat16");
    else if (payload_fp8)
      PSGD_LAUNCH(PSGD_STAGE_QREDUCE, launch_round_fp8_cols(c, 2 * c.nmat, q), "round Q to fp8");
    if (hook && hook(q, p->q_elems, stream, user) != 0) {
      set_error("psgd_compress: aggregation hook failed on Q");
      return PSGD_ERR_HOOK;
    }
  }
  // Aggregated pass-through values back out (with M_hat or the SGD step):
  // extra workgroups of the residual pass on the vector path.
  const bool unpack = mhat || sg.x;
  LaunchCtx c3 = c;
  if (unpack && !c.mfma) c3.unpack_src = pbuf;
  if (!defer_out)
    PSGD_LAUNCH(PSGD_STAGE_RESIDUAL, stage_recon(p, c3, err, q, pbuf, mhat, true, sg), "residual E = M - P_hat Q^T");
  else if (unpack)  // err keeps M; only the decompressed update is written
    PSGD_LAUNCH(PSGD_STAGE_RESIDUAL, stage_recon(p, c3, nullptr, q, pbuf, mhat, false, sg), "decompress P_hat Q^T");
  if (unpack && c.mfma && c.wg_pass > 0)
    PSGD_LAUNCH(PSGD_STAGE_PASSTHRU, launch_pass_unpack(c, pbuf, mhat, sg), "pass-through unpack");
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_compress(psgd_plan_t p, const void* grads, float* err, float* mom, float* q, float* pbuf,
                                       float* mhat, const psgd_step_opts_t* opts, psgd_reduce_fn hook, void* user,
                                       void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  psgd_step_opts_t o;
  if (psgd_status_t s = validate_compress("psgd_compress", p, grads, err, mom, q, pbuf, mhat, opts, &o)) return s;
  if (psgd_status_t s = check_ws(p, ws, ws_bytes, "psgd_compress")) return s;
  return run_compress(p, grads, err, mom, q, pbuf, mhat, o, hook, user, ws, stream);
}

// ------------------------------------------------- allocation-free compress
//
// psgd_compress_noalloc runs the same step with the library's own device
// scratch in place of a caller workspace: one static array per GPU, made when
// the library's code object is loaded on that GPU and kept until the process
// ends.  Its device address is looked up once per device with
// hipGetSymbolAddress; in host code the array's name is only a host-side
// stand-in and is never passed to a kernel or a copy.

static __device__ __align__(256) unsigned char scratch[PSGD_NOALLOC_SCRATCH_BYTES];

namespace psgd {

constexpr int kNoallocMaxDevices = 64;

struct NoallocDevice {
  bool ready = false;            // `ptr` looked up on this device
  void* ptr = nullptr;           // device address of `scratch` on this device
  uint64_t plan_id = 0;          // plan whose tables the scratch holds (0: none)
  hipStream_t stream = nullptr;  // stream those tables were uploaded on
};

static std::mutex g_noalloc_mu;
static NoallocDevice g_noalloc[kNoallocMaxDevices];

}  // namespace psgd

extern "C" psgd_status_t psgd_compress_noalloc(psgd_plan_t p, const void* grads, float* err, float* mom, float* q,
                                               float* pbuf, float* mhat, const psgd_step_opts_t* opts,
                                               psgd_reduce_fn hook, void* user, hipStream_t stream) {
  clear_error();
  psgd_step_opts_t o;
  if (psgd_status_t s = validate_compress("psgd_compress_noalloc", p, grads, err, mom, q, pbuf, mhat, opts, &o))
    return s;
  if ((uint64_t)p->hdr.total_bytes > (uint64_t)PSGD_NOALLOC_SCRATCH_BYTES) {
    set_error("psgd_compress_noalloc: the plan needs %lld bytes of scratch, more than the library's static %lld "
              "(use psgd_compress with a workspace)",
              (long long)p->hdr.total_bytes, (long long)PSGD_NOALLOC_SCRATCH_BYTES);
    return PSGD_ERR_WORKSPACE;
  }
  if (p->ntensors == 0) return PSGD_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "psgd_compress_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kNoallocMaxDevices) {
    set_error("psgd_compress_noalloc: device %d beyond the %d devices supported", dev, kNoallocMaxDevices);
    return PSGD_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    NoallocDevice& st = g_noalloc[dev];
    if (!st.ready) {
      // first call on this device (which is current): the device's own copy
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "psgd_compress_noalloc: hipGetSymbolAddress(scratch)");
      st.ptr = ptr;
      st.ready = true;
    }
    ws = st.ptr;
    // The scratch keeps the last call's contents: the plan's tables are
    // uploaded again whenever another plan (or another stream) used it last.
    if (st.plan_id != p->id || st.stream != stream) {
      st.plan_id = 0;
      if (!p->tables.empty()) {
        e = hipMemcpyAsync(ws, p->tables.data(), p->tables.size(), hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "psgd_compress_noalloc: table upload");
      }
      st.plan_id = p->id;
      st.stream = stream;
    }
  }
  return run_compress(p, grads, err, mom, q, pbuf, mhat, o, hook, user, ws, stream);
}

extern "C" psgd_status_t psgd_decompress(psgd_plan_t p, const float* pbuf, const float* q, float* out, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!p) {
    set_error("psgd_decompress: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (p->ntensors > 0 && (!pbuf || !out || (!p->mats.empty() && !q))) {
    set_error("psgd_decompress: a required buffer is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (!aligned16(pbuf) || !aligned16(q) || !aligned16(out)) {
    set_error("psgd_decompress: buffers must be 16-byte aligned");
    return PSGD_ERR_INVALID_ARG;
  }
  if (psgd_status_t s = check_ws(p, ws, ws_bytes, "psgd_decompress")) return s;
  if (p->ntensors == 0) return PSGD_OK;
  LaunchCtx c = make_ctx(p, ws, stream);
  const SgdArgs none{nullptr, nullptr, 0.f, 0.f};
  if (!c.mfma) c.unpack_src = pbuf;  // pass-through values by extra workgroups of the same launch
  PSGD_LAUNCH(PSGD_STAGE_RESIDUAL, stage_recon(p, c, nullptr, q, pbuf, out, false, none), "decompress P_hat Q^T");
  if (c.mfma && c.wg_pass > 0)
    PSGD_LAUNCH(PSGD_STAGE_PASSTHRU, launch_pass_unpack(c, pbuf, out, none), "pass-through unpack");
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_refresh(psgd_plan_t p, int32_t tensor, const float* m, float* q, int32_t iters, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!p) {
    set_error("psgd_refresh: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (tensor < 0 || tensor >= p->ntensors || p->kind[tensor] != PSGD_KIND_COMPRESSED) {
    set_error("psgd_refresh: tensor %d is not a compressed tensor of the plan", tensor);
    return PSGD_ERR_INVALID_ARG;
  }
  if (!m || !q || !aligned16(m) || !aligned16(q)) {
    set_error("psgd_refresh: m and q must be non-null and 16-byte aligned");
    return PSGD_ERR_INVALID_ARG;
  }
  if (iters < 0) {
    set_error("psgd_refresh: negative iteration count");
    return PSGD_ERR_INVALID_ARG;
  }
  if (psgd_status_t s = check_ws(p, ws, ws_bytes, "psgd_refresh")) return s;
  const size_t k = (size_t)(std::find(p->mat_tensor.begin(), p->mat_tensor.end(), tensor) - p->mat_tensor.begin());
  const LaunchCtx c = make_ctx(p, ws, stream);
  const MatDesc& d = p->mats[k];
  const GridRange rows{d.wg_rows0, p->nrow_wg[k]};
  const GridRange mtp = mat_range(p, k, &MatDesc::wg_mtp0, c.wg_mtp);
  const GridRange red = mat_range(p, k, &MatDesc::wg_red0, c.wg_red);
  const GridRange pred = mat_range(p, k, &MatDesc::wg_pred0, c.wg_pred);
  const int op = c.nmat + (int)k, oq = 2 * c.nmat + (int)k;
  const int nb_p = (d.m + kGramRows - 1) / kGramRows, nb_q = (d.n + kGramRows - 1) / kGramRows;
  float* M = const_cast<float*>(m);
  // Stages are recorded under the step's own stage ids (M Q under EF_P,
  // M^T P under MTP / QREDUCE, orthonormalisations under GS).
  for (int it = 0; it < iters; ++it) {
    PSGD_LAUNCH(PSGD_STAGE_EF_P, stage_mq(p, c, rows, pred, 0, nullptr, M, nullptr, q, c.rscr, 0),
                "refresh: P = M Q");
    PSGD_LAUNCH(PSGD_STAGE_GS, launch_gram_orth(c, op, 1, nullptr, nb_p, c.rscr), "refresh: orthonormalise P");
    {
      StageTimer _t(p, PSGD_STAGE_MTP, stream);
      const hipError_t e = c.mfma ? launch_mfma_qt(c, mtp, M, c.rscr, 0, q) : launch_mtp(c, mtp, M, c.rscr, 0, q);
      if (e != hipSuccess) return hip_fail(e, "refresh: Q = M^T P");
    }
    PSGD_LAUNCH(PSGD_STAGE_QREDUCE, launch_qreduce(c, red, q), "refresh: Q partial reduction");
    PSGD_LAUNCH(PSGD_STAGE_GS, launch_gram_orth(c, oq, 1, nullptr, nb_q, q), "refresh: orthonormalise Q");
  }
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_step_stats(psgd_plan_t p, const float* err, const float* mhat, double* out, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!p) {
    set_error("psgd_step_stats: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (p->mats.empty()) return PSGD_OK;
  if (!err || !mhat || !out || ((uintptr_t)out & 7u)) {
    set_error("psgd_step_stats: err, mhat and out must be non-null (out 8-byte aligned)");
    return PSGD_ERR_INVALID_ARG;
  }
  if (psgd_status_t s = check_ws(p, ws, ws_bytes, "psgd_step_stats")) return s;
  const LaunchCtx c = make_ctx(p, ws, stream);
  const hipError_t e = launch_sumsq(c, err, mhat, out);
  if (e != hipSuccess) return hip_fail(e, "psgd_step_stats");
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_subspace_overlap(psgd_plan_t p, const float* q_a, const float* q_b, float* scratch,
                                               double* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!p) {
    set_error("psgd_subspace_overlap: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (p->mats.empty()) return PSGD_OK;
  if (!q_a || !q_b || !scratch || !out || ((uintptr_t)out & 7u)) {
    set_error("psgd_subspace_overlap: q_a, q_b, scratch and out must be non-null (out 8-byte aligned)");
    return PSGD_ERR_INVALID_ARG;
  }
  const size_t qn = p->q_elems;
  if ((scratch < q_a + qn && q_a < scratch + 2 * qn) || (scratch < q_b + qn && q_b < scratch + 2 * qn)) {
    set_error("psgd_subspace_overlap: scratch must not overlap q_a or q_b");
    return PSGD_ERR_INVALID_ARG;
  }
  if (psgd_status_t s = check_ws(p, ws, ws_bytes, "psgd_subspace_overlap")) return s;
  const LaunchCtx c = make_ctx(p, ws, stream);
  float* a = scratch;
  float* b = scratch + qn;
  hipError_t e = hipMemcpyAsync(a, q_a, qn * sizeof(float), hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(b, q_b, qn * sizeof(float), hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "psgd_subspace_overlap: copy");
  // both copies orthonormalised as the refresh does its Q (Gram-Schmidt with
  // the dependence rule), then the cosines of their principal angles
  const int first = 2 * c.nmat;
  if ((e = launch_gram_orth(c, first, c.nmat, c.gramq_map, c.wg_gramq, a)) != hipSuccess ||
      (e = launch_gram_orth(c, first, c.nmat, c.gramq_map, c.wg_gramq, b)) != hipSuccess)
    return hip_fail(e, "psgd_subspace_overlap: orthonormalise");
  if ((e = launch_overlap(c, first, a, b, out)) != hipSuccess) return hip_fail(e, "psgd_subspace_overlap");
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_init_q(psgd_plan_t p, float* q, uint64_t seed, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  clear_error();
  if (!p) {
    set_error("psgd_init_q: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (!p->mats.empty() && (!q || !aligned16(q))) {
    set_error("psgd_init_q: q must be non-null and 16-byte aligned");
    return PSGD_ERR_INVALID_ARG;
  }
  if (psgd_status_t s = check_ws(p, ws, ws_bytes, "psgd_init_q")) return s;
  if (p->mats.empty()) return PSGD_OK;
  const LaunchCtx c = make_ctx(p, ws, stream);
  int64_t max_blocks = 0;
  for (const MatDesc& d : p->mats) max_blocks = std::max<int64_t>(max_blocks, ((int64_t)d.n * p->rank + 3) / 4);
  const hipError_t e = launch_init_q(c, q, seed, max_blocks);
  if (e != hipSuccess) return hip_fail(e, "psgd_init_q");
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_timing_enable(psgd_plan_t p, int32_t enable) {
  clear_error();
  if (!p) {
    set_error("psgd_timing_enable: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lk(p->timing_mu);
  if (!p->timing) p->timing = new TimingState();
  TimingState* t = p->timing;
  if (enable && !t->reserved) {
    // the pool up front: creating events inside the timed calls would put
    // host work between their launches
    t->pool.reserve(PSGD_TIMING_EVENTS);
    while (t->pool.size() < (size_t)PSGD_TIMING_EVENTS) {
      hipEvent_t e = nullptr;
      const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
      if (err != hipSuccess) {
        t->enabled = false;
        return hip_fail(err, "psgd_timing_enable");
      }
      t->pool.push_back(e);
    }
    t->reserved = true;
  }
  t->enabled = enable != 0;
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_timing_stages(psgd_plan_t p, uint32_t mask) {
  clear_error();
  if (!p) {
    set_error("psgd_timing_stages: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lk(p->timing_mu);
  if (!p->timing) p->timing = new TimingState();
  p->timing->mask = mask;
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_timing_read(psgd_plan_t p, double* ms, int64_t* launches) {
  clear_error();
  if (!p || !ms) {
    set_error("psgd_timing_read: NULL argument");
    return PSGD_ERR_INVALID_ARG;
  }
  for (int i = 0; i < PSGD_NSTAGES; ++i) {
    ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  std::lock_guard<std::mutex> lk(p->timing_mu);
  if (!p->timing) return PSGD_OK;
  psgd_status_t st = PSGD_OK;
  for (TimingRecord& r : p->timing->records) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess && st == PSGD_OK) st = hip_fail(e, "psgd_timing_read");
    ms[r.stage] += t;
    if (launches) launches[r.stage] += 1;
    p->timing->pool.push_back(r.start);
    p->timing->pool.push_back(r.stop);
  }
  p->timing->records.clear();
  return st;
}

extern "C" psgd_status_t psgd_stream_probe(const float* const* in, int32_t nin, float* const* out, int32_t nout,
                                          size_t n, float* sink, hipStream_t stream) {
  clear_error();
  static_assert(PSGD_PROBE_SINK_FLOATS == kProbeSinkFloats, "probe sink size");
  if (nin < 0 || nin > 3 || nout < 0 || nout > 2 || nin + nout == 0 || (nin > 0 && !in) || (nout > 0 && !out) ||
      (nout == 0 && !sink) || (n & 3u)) {
    set_error("psgd_stream_probe: need 0..3 inputs, 0..2 outputs (at least one array), a sink without outputs "
              "and n a multiple of 4 (nin=%d nout=%d n=%zu)", nin, nout, n);
    return PSGD_ERR_INVALID_ARG;
  }
  ProbeArgs a{};
  for (int k = 0; k < nin; ++k) {
    if (!in[k] || !aligned16(in[k])) {
      set_error("psgd_stream_probe: input %d is NULL or not 16-byte aligned", k);
      return PSGD_ERR_INVALID_ARG;
    }
    a.in[k] = reinterpret_cast<const float4*>(in[k]);
  }
  for (int j = 0; j < nout; ++j) {
    if (!out[j] || !aligned16(out[j])) {
      set_error("psgd_stream_probe: output %d is NULL or not 16-byte aligned", j);
      return PSGD_ERR_INVALID_ARG;
    }
    a.out[j] = reinterpret_cast<float4*>(out[j]);
  }
  a.sink = sink;
  a.n4 = (int64_t)(n / 4);
  const hipError_t e = launch_stream_probe(a, nin, nout, stream);
  if (e != hipSuccess) return hip_fail(e, "psgd_stream_probe");
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_stream_copy(float* dst, const float* src, size_t n, hipStream_t stream) {
  clear_error();
  if (!dst || !src || (n & 3u) || ((uintptr_t)dst & 15u) || ((uintptr_t)src & 15u)) {
    set_error("psgd_stream_copy: need 16-byte aligned pointers and n a multiple of 4");
    return PSGD_ERR_INVALID_ARG;
  }
  const hipError_t e = launch_stream_copy(dst, src, n, stream);
  if (e != hipSuccess) return hip_fail(e, "psgd_stream_copy");
  return PSGD_OK;
}
