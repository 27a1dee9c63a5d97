// fa_api.cpp -- the C ABI of libfa_fwd.so: argument validation, the
// shared-memory (LDS) screen, the planner and the launch call.
//
// Everything here except the final fa::launch is plain host arithmetic with
// no HIP call, so every error a caller can make with sizes or pointers is
// reported before the device is touched.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/fa_fwd.h"
#include "fa_internal.h"

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// fa_set_schedule: 0 automatic, else the forced schedule (1 .. 5)
std::atomic<int> g_schedule{0};
// fa_set_exp2_offload: 0, 4 or 8
std::atomic<int> g_exp2_offload{0};
// fa_set_fp8_exact_scores: 0 or 1
std::atomic<int> g_fp8_exact{0};

// gfx950 (MI355X): 160 KiB LDS per CU, all of it addressable by one
// workgroup; 256 CUs; 4 SIMDs per CU; 512 VGPR+AGPR per lane per SIMD;
// 8 wave slots per SIMD.
constexpr fa_device_limits_t kGfx950 = {163840, 163840, 256, 4, 512, 8};

int check_dims(int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k, int head_dim,
               int head_dim_v) {
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || seqlen_q < 0 || seqlen_k < 0 ||
      head_dim <= 0 || head_dim_v <= 0)
    return FA_ERR_INVALID;
  if (heads_q % heads_kv != 0) return FA_ERR_INVALID;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_version(void) { return 100; }

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_INVALID: return "invalid argument (sizes, head ratio or softmax scale)";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration (head dims or no tile plan fits)";
    case FA_ERR_DEVICE: return "device error (not gfx950, or the kernel launch failed)";
    default: return "unknown error code";
  }
}

int fa_check_cu_seqlens(const int* cu, int batch, int seqlen_q, int seqlen_k, int64_t rows_q,
                        int64_t rows_k) {
  if (!cu) return FA_ERR_NULL;
  if (batch <= 0 || seqlen_q < 0 || seqlen_k < 0 || rows_q < 0 || rows_k < 0) return FA_ERR_INVALID;
  const int* ck = cu + batch + 1;
  if (cu[0] != 0 || ck[0] != 0) return FA_ERR_INVALID;
  for (int b = 0; b < batch; ++b) {
    const int64_t lq = (int64_t)cu[b + 1] - cu[b], lk = (int64_t)ck[b + 1] - ck[b];
    if (lq < 0 || lq > seqlen_q || lk < 0 || lk > seqlen_k) return FA_ERR_INVALID;
  }
  if (cu[batch] != rows_q || ck[batch] > rows_k) return FA_ERR_INVALID;
  return FA_OK;
}

int fa_set_schedule(int schedule) {
  if (schedule < 0 || schedule > 5) return FA_ERR_INVALID;
  g_schedule.store(schedule, std::memory_order_relaxed);
  return FA_OK;
}

int fa_set_exp2_offload(int every) {
  if (every != 0 && every != 4 && every != 8) return FA_ERR_INVALID;
  g_exp2_offload.store(every, std::memory_order_relaxed);
  return FA_OK;
}

int fa_set_fp8_exact_scores(int on) {
  if (on != 0 && on != 1) return FA_ERR_INVALID;
  g_fp8_exact.store(on, std::memory_order_relaxed);
  return FA_OK;
}

int fa_gfx950_limits(fa_device_limits_t* out) {
  if (!out) return FA_ERR_NULL;
  *out = kGfx950;
  return FA_OK;
}

// Byte accounting of the shared-memory screen: with Q staged in shared
// memory the Q, K and V tiles add up (K and V once per stage); with Q kept
// in registers after the prologue, the Q buffer and the V buffers have
// disjoint lifetimes and share space, so they combine by max.
int fa_smem_screen(const fa_tile_config_t* cfg, const fa_device_limits_t* dev, fa_screen_t* out) {
  if (!cfg || !dev || !out) return FA_ERR_NULL;
  if (cfg->tile_m <= 0 || cfg->tile_n <= 0 || cfg->head_dim <= 0 || cfg->head_dim_v <= 0 ||
      cfg->elem_bytes <= 0 || cfg->kv_stages <= 0 || dev->lds_bytes_per_block <= 0 ||
      dev->lds_bytes_per_cu <= 0)
    return FA_ERR_INVALID;
  const int64_t e = cfg->elem_bytes;
  const int64_t q = (int64_t)cfg->tile_m * cfg->head_dim * e;
  const int64_t k = (int64_t)cfg->tile_n * cfg->head_dim * e * cfg->kv_stages;
  const int64_t v = (int64_t)cfg->tile_n * cfg->head_dim_v * e * cfg->kv_stages;
  out->smem_bytes = cfg->q_in_regs ? k + (q > v ? q : v) : q + k + v;
  out->fits = out->smem_bytes <= dev->lds_bytes_per_block;
  out->blocks_per_cu = out->fits ? (int)(dev->lds_bytes_per_cu / out->smem_bytes) : 0;
  return FA_OK;
}

int fa_fwd_plan(int dtype, int batch, int heads_q, int heads_kv, int seqlen_q, int seqlen_k,
                int varlen, int head_dim, int head_dim_v, int causal,
                const fa_device_limits_t* dev, fa_plan_t* out) {
  if (!out) return FA_ERR_NULL;
  int rc = check_dims(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, head_dim_v);
  if (rc) return rc;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_E4M3) return FA_ERR_INVALID;
  if ((head_dim != 64 && head_dim != 128) || head_dim_v != head_dim) return FA_ERR_UNSUPPORTED;
  const fa_device_limits_t& L = dev ? *dev : kGfx950;
  if (L.lds_bytes_per_block <= 0 || L.lds_bytes_per_cu <= 0 || L.simds_per_cu <= 0 ||
      L.regs_per_simd_lane <= 0)
    return FA_ERR_INVALID;
  // The compiled kernels (64-key blocks, Q in registers, K/V double-buffered
  // in LDS without padding):
  //  * schedule 1: 4 waves, one 32-row query tile each: 128 rows of one head
  //    per workgroup, 256 registers per lane (2 waves per SIMD);
  //  * schedule 2 (bf16): 4 waves with two query tiles each: 256 rows of one
  //    head, the full 512-register file (1 wave per SIMD); each LDS operand
  //    read feeds two MFMAs;
  //  * schedule 3 (bf16, heads_q / heads_kv even, or odd without varlen): 8
  //    waves in two groups of four, 128 rows of two query heads that share a
  //    KV head -- or, for an odd heads_q / heads_kv (1: MHA), two adjacent
  //    128-row tiles of one head --,
  //    alternating GEMM and softmax slots (ping-pong), 256 registers per lane;
  //  * schedule 5 (forced only, where 3 applies): the items of schedule 3
  //    walked by resident workgroups (one per CU), each taking its XCD's
  //    items in zig-zag windows and prefetching the next item's query rows
  //    into an LDS stage before the current item's epilogue;
  //  * schedule 4 (bf16, heads_q / heads_kv * seqlen_q <= 32): decode -- all
  //    query rows of one KV head's group in the 32 columns of one tile, one
  //    workgroup per (sequence, KV head) whose 4 waves split the key range in
  //    32-key blocks, each with a 2-slot K and V ring in LDS, one wave per
  //    SIMD.
  // Automatic: 4 where it applies, else 3 where it applies with at least one
  // workgroup per CU, else 1.
  // fa_set_schedule forces one (falling back to 1 where it does not apply).
  const int64_t lds = fa::lds_bytes(head_dim, dtype == FA_DTYPE_E4M3 ? 1 : 2);
  if (lds > L.lds_bytes_per_block) return FA_ERR_UNSUPPORTED;
  const int64_t pairs = (int64_t)batch * heads_kv;
  const int group = heads_q / heads_kv;
  const bool bf16 = dtype == FA_DTYPE_BF16;
  const bool wide_ok = bf16 && L.regs_per_simd_lane >= 512;
  // Odd groups (MHA) take the ping-pong as tile pairs only for fixed lengths: on packed
  // varlen batches the 256-row granularity (half-empty last pairs, the lower
  // tile's masked blocks on every diagonal) measured 5 % slower than
  // schedule 1's two 128-row workgroups per CU
  const bool pp_ok = bf16 && (group % 2 == 0 || !varlen) &&
                     L.regs_per_simd_lane >= 512;
  // The ping-pong kernel puts twice the rows of schedule 1 into a workgroup
  // (and one workgroup on a CU): where that leaves CUs idle, schedule 1's
  // finer grid finishes first (the 2-head x 256-row case measured 8.6 us
  // against 6.2 us), so the automatic choice takes it only for grids of at
  // least one workgroup per CU -- or, without causal masking, for more than
  // half a round: there schedule 1's twice as many workgroups put two on
  // some CUs, and the ping-pong measured +14 to +20 % (160-192 workgroups on
  // 256 CUs, MHA and GQA, 1536-6144 rows; -14 to -16 % at exactly 128).
  // Causal grids below a round stay on schedule 1 (0 to -19 % for the
  // ping-pong).
  const int64_t pp_rows = group % 2 ? 2LL * fa::kTileM : fa::kTileM;
  const int64_t pp_items = (int64_t)batch * heads_kv * (group % 2 ? group : group / 2) *
                           ((seqlen_q + pp_rows - 1) / pp_rows);
  // Causal tile pairs give the lower tile two fully masked key blocks per
  // pair; measured against schedule 1 (head_dim 128) they win from 6144 rows
  // (+5 to +13 % at 6144, +8 to +16 % at 8192-16384) and on a single round of
  // pairs (MHA 4 x 16 x 1024: +10 %), and lose at 2048-4096 rows over several
  // rounds (-2 to -3 %, +5 % for 1024 items); non-causal pairs win (+9 to +20 %).
  // Short causal sequences (below 2048 rows) over several rounds favour
  // schedule 1 for head pairs too (GQA 32/8 causal at 512-1536 rows: -1 to
  // -16 %; 2048: +1.7 %; 4096: +3.4 %): its two workgroups per CU overlap
  // each other's tile starts.  Without causal masking the ping-pong wins from
  // 1024 rows (+3 to +8 % on seven of nine MHA, GQA and group-3 shapes at
  // 1024-1536 rows, -4 % on the other two; 512-768 rows: -4 to -7 %).
  const bool one_round = pp_items <= L.num_cus;
  const bool pairs_ok = group % 2 == 0 || !causal || seqlen_q >= 6144 || one_round;
  // A single causal round over at most kXcds (sequence, KV head) pairs: its
  // critical path is the heaviest item, which schedule 1 finishes 6-11 %
  // sooner (one sequence with 1, 4 or 8 KV heads, 1024-8192 rows, head pairs
  // and tile pairs alike); with 16 or more pairs the ping-pong wins (+9 to
  // +13 %).
  const bool few_pairs_round = causal && one_round && pairs <= fa::kXcds;
  // At head_dim 64 a key block carries half the matrix work of head_dim 128
  // beside the same softmax, and the ping-pong measured slower than schedule 1
  // on every shape tried (head pairs and tile pairs, causal or not, 1024-16384
  // rows: -0.3 to -30 %, typically -4 to -10 %): it is taken for head_dim 128
  // only.
  const bool pp_dim = head_dim == 128;
  const bool pp_fill = pp_items >= L.num_cus || (!causal && 2 * pp_items > L.num_cus);
  const bool pp_auto = pp_ok && pp_dim && pp_fill && pairs_ok &&
                       (seqlen_q >= (causal ? 2048 : 1024) || one_round) && !few_pairs_round;
  // each wave's ring of K and V slots of 32 keys
  const int64_t decode_lds = (int64_t)fa::kDecodeWaves * fa::kDecodeSlots * 2 * 32 * head_dim * 2;
  const bool decode_ok = bf16 && (int64_t)group * seqlen_q <= 32 && seqlen_q > 0 &&
                         L.regs_per_simd_lane >= 512 && decode_lds <= L.lds_bytes_per_block;
  const int forced = g_schedule.load(std::memory_order_relaxed);
  int sched = forced ? forced : (decode_ok ? 4 : pp_auto ? 3 : 1);
  // schedule 5: the ping-pong items walked by resident workgroups, with a Q
  // stage for the next item's rows beside the K/V stages
  const int64_t q_stage = 2LL * fa::kWaves * 32 * head_dim * 2;
  const bool persist_ok = pp_ok && lds + q_stage <= L.lds_bytes_per_block && L.num_cus >= fa::kXcds;
  if ((sched == 2 && !wide_ok) || (sched == 3 && !pp_ok) || (sched == 4 && !decode_ok) ||
      (sched == 5 && !persist_ok))
    sched = 1;
  if (sched == 4) {
    out->tile_m = 32;  // (query head, row) columns of one tile
    out->tile_n = 32;
    out->waves = fa::kDecodeWaves;
    out->kv_stages = fa::kDecodeSlots;
    out->lds_bytes = decode_lds;
    out->wg_per_cu = 1;
    out->vgprs_per_lane = 512;
    out->query_tiles = 1;
    out->heads_per_workgroup = group;
    out->schedule = 4;
    out->m_tiles = seqlen_q > 0 ? 1 : 0;
    out->num_workgroups = out->m_tiles == 0 ? 0 : (int64_t)batch * heads_kv;
    out->kernel_variant = (head_dim == 128 ? 0 : 2) + (causal ? 1 : 0);
    return FA_OK;
  }
  const int qt = sched == 2 ? 2 : 1;
  const bool pp = sched == 3 || sched == 5;
  const int waves = pp ? 2 * fa::kWaves : fa::kWaves;
  // schedules 3 and 5 with an odd heads_q / heads_kv: two adjacent 128-row
  // tiles of one head per workgroup instead of two heads
  const bool mpair = pp && group % 2 == 1;
  const int heads_per_wg = pp && !mpair ? 2 : 1;
  const int vgprs = 256 * qt;
  const int by_regs = (L.regs_per_simd_lane / vgprs) * L.simds_per_cu / waves;
  out->tile_m = fa::kTileM * (mpair ? 2 : qt);
  out->tile_n = fa::kTileN;
  out->waves = waves;
  out->kv_stages = fa::kStages;
  out->lds_bytes = sched == 5 ? lds + q_stage : lds;
  const int by_lds_s = (int)(L.lds_bytes_per_cu / out->lds_bytes);
  out->wg_per_cu = by_lds_s < by_regs ? by_lds_s : by_regs;
  out->vgprs_per_lane = vgprs;
  out->query_tiles = qt;
  out->heads_per_workgroup = heads_per_wg;
  out->schedule = sched;
  out->m_tiles = (seqlen_q + out->tile_m - 1) / out->tile_m;
  // one slot per (query tile, query head or head pair) of every (sequence,
  // kv-head) pair: whole rounds of kXcds pairs dealt to the XCDs, the other
  // pairs' items spread over all of them (fa::prefill_grid)
  out->num_workgroups = out->m_tiles == 0 ? 0
                        : fa::prefill_grid(pairs, out->m_tiles, group / heads_per_wg).workgroups;
  if (sched == 5) {  // resident workgroups: one per CU, a whole number per XCD, at most one per item
    const int64_t resident = (int64_t)(L.num_cus / fa::kXcds) * fa::kXcds;
    if (out->num_workgroups > resident) out->num_workgroups = resident;
  }
  out->kernel_variant = (head_dim == 128 ? 0 : 2) + (causal ? 1 : 0) + (dtype == FA_DTYPE_E4M3 ? 4 : 0);
  if (out->wg_per_cu <= 0) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // extern "C"

namespace {

// The forward launch shared by fa_fwd and fa_fwd_kvcache.  cache_seqlens ==
// NULL: K/V rows per sequence as fa_fwd documents; else the KV-cache mode
// (fixed-length layout with seqlen_k = cache capacity, cu_seqlens NULL).
int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                 int heads_q, int heads_kv, int seqlen_q, int seqlen_k, const int* cu_seqlens,
                 const int* cache_seqlens, int seqlen_new, int head_dim, int head_dim_v,
                 float softmax_scale, int causal, const float* descales, void* stream) {
  int rc = check_dims(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, head_dim_v);
  if (rc) return rc;
  // Q/O/LSE may be NULL only when there is no query row, K/V only when there
  // is no key: a zero length, for a packed batch a zero maximum (every
  // sequence's length is at most the maximum passed).
  if ((!q || !o || !lse) && seqlen_q > 0) return FA_ERR_NULL;
  if ((!k || !v) && seqlen_k > 0) return FA_ERR_NULL;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  const int dtype = descales ? FA_DTYPE_E4M3 : FA_DTYPE_BF16;
  fa_plan_t plan;
  rc = fa_fwd_plan(dtype, batch, heads_q, heads_kv, seqlen_q, seqlen_k, cu_seqlens != nullptr,
                   head_dim, head_dim_v, causal, nullptr, &plan);
  if (rc) return rc;
  if (plan.num_workgroups > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  const int qt = plan.query_tiles;
  // The kernel addresses one sequence's K or V through a buffer resource
  // whose byte range is a 31-bit quantity.
  const int64_t elem = dtype == FA_DTYPE_E4M3 ? 1 : 2;
  if ((int64_t)seqlen_k * heads_kv * head_dim * elem >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  // sequence offsets (rows) are 32-bit in the kernel
  if (!cu_seqlens && ((int64_t)batch * seqlen_q >= (1LL << 31) ||
                      (int64_t)batch * seqlen_k >= (1LL << 31)))
    return FA_ERR_UNSUPPORTED;
  if (plan.num_workgroups == 0) return FA_OK;  // no query rows: nothing to write
  fa::Launch L;
  L.p.q = q;
  L.p.k = k;
  L.p.v = v;
  L.p.o = o;
  L.p.lse = lse;
  L.p.cu = cu_seqlens;
  L.p.descales = descales;
  L.p.cache_seqlens = cache_seqlens;
  L.p.seqlen_new = seqlen_new;
  L.p.batch = batch;
  L.p.hq = heads_q;
  L.p.hkv = heads_kv;
  L.p.group = heads_q / heads_kv;
  L.p.seqlen_q = seqlen_q;
  L.p.seqlen_k = seqlen_k;
  L.p.m_tiles = plan.m_tiles;
  if (plan.schedule != 4) {
    const fa::Grid gr = fa::prefill_grid((int64_t)batch * heads_kv, plan.m_tiles,
                                         (heads_q / heads_kv) / plan.heads_per_workgroup);
    L.p.full_pairs = (int)gr.full_pairs;
    L.p.lin_items = (int)gr.lin_items;
  } else {
    L.p.full_pairs = L.p.lin_items = 0;
  }
  L.p.scale_log2 = softmax_scale * kLog2e;
  L.head_dim = head_dim;
  L.causal = causal;
  L.fp8 = dtype == FA_DTYPE_E4M3;
  L.num_workgroups = plan.num_workgroups;
  L.query_tiles = qt;
  L.pingpong = plan.schedule == 3 || plan.schedule == 5;
  L.persist = plan.schedule == 5;
  // the items of the one-item kernel's grid, walked by the resident workgroups
  L.num_items = L.persist ? fa::prefill_grid((int64_t)batch * heads_kv, plan.m_tiles,
                                             (heads_q / heads_kv) / plan.heads_per_workgroup)
                                .workgroups
                          : plan.num_workgroups;
  L.decode = plan.schedule == 4;
  L.exp2_offload = L.pingpong ? g_exp2_offload.load(std::memory_order_relaxed) : 0;
  L.fp8_exact = L.fp8 ? g_fp8_exact.load(std::memory_order_relaxed) : 0;
  return fa::launch(L, stream);
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
           int heads_q, int heads_kv, int seqlen_q, int seqlen_k, const int* cu_seqlens,
           int head_dim, int head_dim_v, float softmax_scale, int causal, const float* descales,
           void* stream) {
  return forward_impl(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k, cu_seqlens,
                      nullptr, 0, head_dim, head_dim_v, softmax_scale, causal, descales, stream);
}

int fa_fwd_kvcache(const void* q, void* k_cache, void* v_cache, const void* k_new,
                   const void* v_new, void* o, float* lse, int batch, int heads_q, int heads_kv,
                   int seqlen_q, int seqlen_new, int cache_capacity, const int* cache_seqlens,
                   int head_dim, int head_dim_v, float softmax_scale, int causal,
                   const float* descales, void* stream) {
  if (seqlen_new < 0 || cache_capacity < 0) return FA_ERR_INVALID;
  int rc = check_dims(batch, heads_q, heads_kv, seqlen_q, cache_capacity, head_dim, head_dim_v);
  if (rc) return rc;
  if (!cache_seqlens) return FA_ERR_NULL;
  if ((!k_new || !v_new) && seqlen_new > 0) return FA_ERR_NULL;
  if ((!k_cache || !v_cache) && cache_capacity > 0) return FA_ERR_NULL;
  if ((head_dim != 64 && head_dim != 128) || head_dim_v != head_dim) return FA_ERR_UNSUPPORTED;
  const int64_t elem = descales ? 1 : 2;
  if ((int64_t)cache_capacity * heads_kv * head_dim * elem >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  if ((int64_t)batch * seqlen_new * heads_kv * head_dim * elem >= (1LL << 40)) return FA_ERR_UNSUPPORTED;
  // validate the forward's own arguments before anything is written
  if ((!q || !o || !lse) && seqlen_q > 0) return FA_ERR_NULL;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (seqlen_new > 0 && cache_capacity > 0) {
    fa::Append A;
    A.k_cache = k_cache;
    A.v_cache = v_cache;
    A.k_new = k_new;
    A.v_new = v_new;
    A.cache_seqlens = cache_seqlens;
    A.batch = batch;
    A.seqlen_new = seqlen_new;
    A.capacity = cache_capacity;
    A.row_bytes = (int)(heads_kv * head_dim * elem);
    rc = fa::launch_append(A, stream);
    if (rc) return rc;
  }
  return forward_impl(q, k_cache, v_cache, o, lse, batch, heads_q, heads_kv, seqlen_q,
                      cache_capacity, nullptr, cache_seqlens, seqlen_new, head_dim, head_dim_v,
                      softmax_scale, causal, descales, stream);
}

}  // extern "C"
