// fa_internal.h -- what the C-ABI layer (fa_api.cpp) hands to the kernel
// launcher (fa_fwd_kernel.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

namespace fa {

// Kernel geometry shared by the planner and the launcher.
constexpr int kTileM = 128;  // query rows per workgroup per query tile (4 waves x 32 rows)
constexpr int kTileN = 64;   // keys per main-loop step
constexpr int kWaves = 4;    // wavefronts per workgroup
constexpr int kStages = 2;   // K/V LDS buffers
constexpr int kXcds = 8;     // XCDs of an MI355X; workgroups go round-robin over them
#ifndef DEC_SLOTS
#define DEC_SLOTS 2
#endif
#ifndef DEC_WAVES
#define DEC_WAVES 4
#endif
constexpr int kDecodeSlots = DEC_SLOTS;  // K and V LDS ring slots per wave of the decode kernel
constexpr int kDecodeWaves = DEC_WAVES;  // waves of the decode kernel (they split the keys)

// LDS per workgroup: K and V blocks of kTileN rows of d*2 bytes (no padding;
// bank conflicts are avoided by swizzling 16-byte columns), double-buffered.
constexpr int64_t lds_bytes(int d, int elem_bytes) {
  return (int64_t)kStages * 2 * kTileN * d * elem_bytes;
}

// Grid of a prefill schedule with `slots` workgroups per (query tile, pair):
// the items of the pairs beyond whole rounds of kXcds first (padded to a
// multiple of kXcds), then whole rounds dealt to the XCDs.
struct Grid {
  int64_t full_pairs, lin_items, workgroups;
};
constexpr Grid prefill_grid(int64_t pairs, int64_t m_tiles, int64_t slots) {
  const int64_t full = pairs / kXcds * kXcds;
  const int64_t lin = (pairs - full) * m_tiles * slots;
  const int64_t lin_padded = (lin + kXcds - 1) / kXcds * kXcds;
  return Grid{full, lin_padded, lin_padded + full * m_tiles * slots};
}

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* cu;          // NULL or int32[2*(batch+1)]
  const float* descales;  // NULL or float[3]
  // KV-cache mode (cu == NULL): sequence b's keys are rows b*seqlen_k ..
  // of K/V (seqlen_k = cache capacity), of which the first
  // min(cache_seqlens[b] + seqlen_new, seqlen_k) are used
  const int* cache_seqlens;
  int seqlen_new;
  int batch, hq, hkv, group, seqlen_q, seqlen_k;
  int m_tiles;            // query tiles per (sequence, head)
  // grid layout: the pairs of whole rounds of kXcds (full_pairs of them) are
  // dealt to the XCDs after the first lin_items ids, which spread the items
  // of the remaining pairs over all XCDs (a multiple of kXcds)
  int full_pairs, lin_items;
  float scale_log2;       // softmax_scale * log2(e)
};

struct Launch {
  Params p;
  int head_dim;
  int causal;
  int fp8;
  int query_tiles;  // 32-row query tiles per wave (1 or 2)
  int pingpong;     // 1: the 8-wave ping-pong kernel (bf16, two query heads per workgroup)
  int decode;       // 1: the decode kernel (bf16, a KV head's query rows in one tile)
  int exp2_offload; // ping-pong only: 0, or every 4th / 8th exponential on the FMA polynomial
  int persist;      // ping-pong only: 1 for the persistent kernel (num_items items)
  int fp8_exact;    // fp8 only: 1 for scores on the bf16 MFMA from widened Q and K
  int64_t num_items;
  int64_t num_workgroups;
};

// Returns 0, or FA_ERR_DEVICE when the device is not gfx950 or the launch fails.
int launch(const Launch& L, void* stream);

// Appending new K/V rows to a KV cache: rows [b][j] (j < seqlen_new) of
// k_new / v_new go to rows [b][cache_seqlens[b] + j] of the caches; rows
// whose position falls outside [0, capacity) are skipped.
struct Append {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  const int* cache_seqlens;
  int batch, seqlen_new, capacity;
  int row_bytes;  // heads_kv * head_dim * element bytes (a multiple of 16)
};

// Same return convention as launch().
int launch_append(const Append& A, void* stream);

}  // namespace fa
