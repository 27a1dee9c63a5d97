// fa_fwd_kernel.hip -- exact attention forward for gfx950 (MI355X, CDNA4).
//
// Five schedules of one computation (the planner in fa_api.cpp picks one):
//  1. fa_fwd_bf16_kernel<.., QG = 1> / fa_fwd_fp8_kernel: 4 waves = 128 query
//     rows of one (sequence, head), two workgroups per CU;
//  2. fa_fwd_bf16_kernel<.., QG = 2>: 256 rows, one wave per SIMD;
//  3. fa_fwd_bf16_pp_kernel: 8 waves, two query heads of one KV head (or,
//     with an odd number of query heads per KV head, two adjacent query tiles of one), the
//     two groups of waves alternating GEMM and softmax phases (ping-pong);
//  4. fa_fwd_bf16_decode_kernel: a KV head's (query head, row) pairs in one
//     32-column tile, the waves (DEC_WAVES, 4) splitting the key range;
//  5. fa_fwd_bf16_pp_persist_kernel (forced only): schedule 3's items walked
//     by resident workgroups that prefetch their next item's query rows.
// fa_fwd_fp8_kernel<.., XS = true> is the e4m3 kernel with its scores on the
// bf16 matrix instruction from exactly widened Q and K (opt-in).
// The description below is that of schedule 1; the others say how they
// differ.  One workgroup = 4 wavefronts = 128 query rows of one (sequence,
// head).  Each wave owns 32 query rows and walks the key blocks (64 keys
// each) from the last admissible block down to the first, the block order of
// the consumer loop in "FlashAttention core algorithm: forward pass".
//
// Per key block n the wave computes, on the matrix cores, the transposed
// score tile S^T = K_n Q^T (v_mfma_f32_32x32x16_bf16, fp32 accumulate), so
// that every lane holds scores of ONE query (lane % 32) against 32 keys and
// the row max / row sum are in-lane reductions plus one permlane32_swap
// between the two half-waves.  The online softmax runs in exp2 form with the
// scale folded into one constant (softmax_scale * log2 e), as the page's
// softmax_scale_log2 does, then O^T += V_n^T P^T reuses the exp'd score
// accumulator directly as the B operand (no data movement): the K rows are
// written into LDS in an order that makes the accumulator's key order equal
// the operand order the second product expects.  V stays row-major in LDS
// and is read transposed with ds_read_b64_tr_b16.
//
// K/V blocks are double-buffered in LDS and loaded one block ahead by
// buffer loads that write LDS directly, so one barrier per block suffices
// (each wave waits for its own loads before it).  The epilogue normalises by
// the row sum, writes O (bf16) and LSE (fp32, natural log), and writes
// O = 0 / LSE = -inf for rows with no admissible key -- the store_zero path
// of the page's epilogue.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/fa_fwd.h"
#include "fa_exp2_poly.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum that propagates NaN (IEEE 754-2019 maximum).  Scores are never NaN
// here; unlike fmaxf it needs no quieting of its inputs, and chains of it map
// onto v_maximum3_f32.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum of the 32 scores a lane holds for one key block (two 16-register
// accumulators), as four independent chains of three-input maxima.
__device__ __forceinline__ float block_max(const f32x16 (&s)[2]) {
  float ch[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x16& v = s[q >> 1];
    const int r0 = 8 * (q & 1);
    float m = fmax_nan(v[r0], v[r0 + 1]);
#pragma unroll
    for (int j = 2; j < 8; j += 2) m = fmax_nan(fmax_nan(m, v[r0 + j]), v[r0 + j + 1]);
    ch[q] = m;
  }
  return fmax_nan(fmax_nan(ch[0], ch[1]), fmax_nan(ch[2], ch[3]));
}

// max / sum of a value over lanes l and l^32 (the two half-waves hold the
// same 32 queries): permlane32_swap returns {own, partner} in some order.
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS row of key `row` (0..63) of a K block: bits 2 and 3 swapped.  With this
// order, accumulator register r of lane (l%32, half h) in 32-key sub-tile t
// holds key 32t + 16(r/8) + 8h + r%8, which is exactly the key that the B
// operand of the P V product expects in slot r%8 of k-chunk 2t + r/8.
__device__ __forceinline__ int k_lds_row(int row) {
  return row ^ ((((row >> 2) ^ (row >> 3)) & 1) * 12);
}

struct SeqInfo {
  int q0, sq, k0, sk, total_q;
};

__device__ __forceinline__ SeqInfo seq_info(const Params& p, int b) {
  SeqInfo s;
  if (p.cu) {
    s.q0 = p.cu[b];
    s.sq = p.cu[b + 1] - s.q0;
    s.k0 = p.cu[p.batch + 1 + b];
    s.sk = p.cu[p.batch + 2 + b] - s.k0;
    s.total_q = p.cu[p.batch];
  } else {
    s.q0 = b * p.seqlen_q;
    s.sq = p.seqlen_q;
    s.k0 = b * p.seqlen_k;
    s.sk = p.seqlen_k;
    s.total_q = p.batch * p.seqlen_q;
    if (p.cache_seqlens) s.sk = max(0, min(p.cache_seqlens[b] + p.seqlen_new, p.seqlen_k));
  }
  return s;
}

// The work item of a prefill workgroup: (sequence, KV head) pair, query tile
// counted from the heaviest (mrev; the last tile under causal masking), and
// head slot within the pair (hsub < hslots).  Workgroups are dispatched
// round-robin over the XCDs (block id mod kXcds), each XCD with its own L2.
// Whole rounds of kXcds pairs are dealt to the XCDs (pair = xcd + kXcds*k):
// an XCD works through its pairs one at a time, heaviest query tiles first,
// all head slots side by side, so the workgroups resident on one XCD share
// one pair's K/V in its L2.  The pairs left over from whole rounds (all of
// them when there are fewer than kXcds, e.g. one sequence with a few KV
// heads) would leave XCDs idle that way; their items come first in the grid
// instead, heaviest tiles of every such pair first, spread over all XCDs
// (p.lin_items ids, padded to a multiple of kXcds so that the dealt part
// keeps block id mod kXcds = XCD).  False for padding.
struct ItemIdx {
  int pair, mrev, hsub;
};
__device__ __forceinline__ bool item_index(const Params& p, const unsigned id, const int hslots,
                                           ItemIdx& it) {
  if ((int)id < p.lin_items) {
    const int per_tile = (p.batch * p.hkv - p.full_pairs) * hslots;
    it.mrev = (int)id / per_tile;
    const int rem = (int)id - it.mrev * per_tile;
    it.pair = p.full_pairs + rem / hslots;
    it.hsub = rem - (rem / hslots) * hslots;
    return it.mrev < p.m_tiles;
  }
  const unsigned id2 = id - (unsigned)p.lin_items;
  const int xcd = id2 % kXcds;
  const int slot = id2 / kXcds;
  const int per_pair = p.m_tiles * hslots;
  const int kk = slot / per_pair;
  const int within = slot - kk * per_pair;
  it.pair = xcd + kXcds * kk;
  it.mrev = within / hslots;
  it.hsub = within - it.mrev * hslots;
  return it.pair < p.full_pairs;
}

// A row max may grow by up to kLazy (in exp2 units) before O and l are
// rescaled: P then stays <= 2^kLazy = kLazyBound, and O / l is unchanged
// because both are taken relative to the same stale maximum.
constexpr float kLazy = 8.f;
constexpr float kLazyBound = 256.f;

// Instruction classes of the scheduling hints (LLVM AMDGPU sched_group_barrier
// masks); the hints only order instructions the compiler already emits.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedTrans = 0x400;
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// Buffer resource word 3 for raw (untyped, unswizzled) gfx9 buffer loads.
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void;

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Pin MFMA results before divergent code.  An MFMA reads operands from all 64
// lanes; if the compiler sinks one below a branch on a per-lane condition (the
// epilogue's "row exists" test), the lanes switched off there feed it zeros.
// An empty asm that consumes the accumulators keeps every MFMA that produces
// them above this point, under the full execution mask.  (The lambdas that
// call it are also compiled for the host, where it is empty.)
template <int N>
__host__ __device__ __forceinline__ void pin_accumulators(f32x16 (&acc)[N]) {
#if __HIP_DEVICE_COMPILE__
#pragma unroll
  for (int i = 0; i < N; ++i) __asm__ volatile("" : "+v"(acc[i]));
#endif
}
// The same for accumulators that live in AGPRs (kernels that use the full
// 512-register file): an "a" constraint keeps the register allocator from
// homing them in VGPRs and copying them across every loop iteration.
template <int N>
__host__ __device__ __forceinline__ void pin_accumulators_agpr(f32x16 (&acc)[N]) {
#if __HIP_DEVICE_COMPILE__
#pragma unroll
  for (int i = 0; i < N; ++i) __asm__ volatile("" : "+a"(acc[i]));
#endif
}

// O rows out of the O^T accumulator tiles.  Lane (query, hf) holds dims
// 32t + 8i + 4hf + 0..3 of its query's row; one swap across the half-waves per
// dword gives the low lane dims 32t + 16j + 0..7 and the high lane dims
// 32t + 16j + 8..15, so every lane stores 16 contiguous bytes (half the store
// instructions and twice the bytes per row per instruction of 8-byte stores).
// All 64 lanes must be active (the two lanes of a query share `valid`).
template <int DT>
__device__ __forceinline__ void store_o_rows(const f32x16 (&acc)[DT], float scale, __bf16* row,
                                             int hf, bool valid) {
  u32x4 ost[DT][2];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x4 e, f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        e[x] = (__bf16)(acc[t][8 * j + x] * scale);
        f[x] = (__bf16)(acc[t][8 * j + 4 + x] * scale);
      }
      u32x2 eu = __builtin_bit_cast(u32x2, e), fu = __builtin_bit_cast(u32x2, f);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const auto r = __builtin_amdgcn_permlane32_swap(eu[w], fu[w], false, false);
        eu[w] = r[0];
        fu[w] = r[1];
      }
      ost[t][j] = u32x4{eu[0], eu[1], fu[0], fu[1]};
    }
  if (valid) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) *(u32x4*)(row + 32 * t + 16 * j + 8 * hf) = ost[t][j];
  }
}

// LDS layout of a 64-key block (K or V): 64 rows of D*2 bytes, no padding.
// 16-byte column `lc` of row `r` is stored at physical column lc ^ swz(r):
//  * K rows are read 16 B per lane by 16 consecutive rows at one column per
//    LDS cycle, so swz_k makes those 16 rows hit 16 different 16-byte bank
//    groups (256 B = all 64 banks);
//  * V rows are read by the transposing 8-byte loads, four consecutive rows x
//    64 contiguous bytes per half-wave, so swz_v spreads the four rows over
//    the four 64-byte quarters of the bank space.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// QG = query groups of 32 rows per wave.  QG = 1: 128 rows per workgroup,
// two workgroups (eight waves) per CU.  QG = 2: 256 rows per workgroup, one
// wave per SIMD with the full 512-register file; every K operand read and
// every transposed V read from LDS then feeds two MFMAs instead of one, which
// halves the LDS traffic per MFMA (the transposed V reads are what limits the
// QG = 1 tiling).
template <int D, bool CAUSAL, int QG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QG == 1 ? 2 : 1, QG == 1 ? 2 : 1)))
void fa_fwd_bf16_kernel(Params p) {
  constexpr int TM = kTileM * QG, TN = kTileN;
  constexpr int RB = D * 2;                  // bytes per K/V row in LDS
  constexpr int BUF = TN * RB;               // bytes per K or V block buffer
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NI = TN * CPR / 256;         // direct-load instructions per wave per block
  constexpr int KC = D / 16;                 // k-chunks of the QK^T product
  constexpr int DT = D / 32;                 // 32-wide output tiles of O^T
  // LDS: K buffers [2][TN rows], then V buffers [2][TN rows]
  __shared__ __attribute__((aligned(1024))) char smem[4 * BUF];
  char* const kbuf0 = smem;
  char* const vbuf0 = smem + 2 * BUF;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  // ---- work item: one query head per head slot
  ItemIdx itx;
  if (!item_index(p, blockIdx.x, p.group, itx)) return;  // padding
  const int pair = itx.pair, mrev = itx.mrev;
  const int b = pair / p.hkv;
  const int head = (pair - b * p.hkv) * p.group + itx.hsub;
  const int mblk = CAUSAL ? (p.m_tiles - 1 - mrev) : mrev;
  const SeqInfo si = seq_info(p, b);
  const int m0 = mblk * TM;
  if (m0 >= si.sq) return;  // uniform over the workgroup, before any barrier
  const int g = head / p.group;
  int qi[QG];       // this lane's query rows in the sequence (one per group)
  bool qvalid[QG];
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    qi[q] = m0 + (wave * QG + q) * 32 + r32;
    qvalid[q] = qi[q] < si.sq;
  }

  const __bf16* __restrict__ Q = (const __bf16*)p.q;
  __bf16* __restrict__ O = (__bf16*)p.o;
  const float c = p.scale_log2;

  // ---- number of key blocks this tile needs
  const int diag = si.sk - si.sq;  // bottom-right alignment offset
  int kend = si.sk;
  if (CAUSAL) kend = min(kend, m0 + TM + diag);
  const int nblk = kend > 0 ? (kend + TN - 1) / TN : 0;

  int64_t orow[QG], lse_idx[QG];
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    orow[q] = ((int64_t)(si.q0 + qi[q]) * p.hq + head) * D;
    lse_idx[q] = (int64_t)head * si.total_q + si.q0 + qi[q];
  }

  if (nblk == 0) {  // no admissible key for any row of the tile: store_zero
#pragma unroll
    for (int q = 0; q < QG; ++q)
      if (qvalid[q]) {
        for (int e = hf * 4; e < D; e += 8) *(u32x2*)(O + orow[q] + e) = u32x2{0u, 0u};
        if (hf == 0) p.lse[lse_idx[q]] = -INFINITY;
      }
    return;
  }

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[qi][16kc + 8hf .. +7]
  bf16x8 qf[QG][KC];
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    const __bf16* qp = Q + orow[q] + 8 * hf;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 t = qvalid[q] ? *(const u32x4*)(qp + 16 * kc) : u32x4{0u, 0u, 0u, 0u};
      qf[q][kc] = __builtin_bit_cast(bf16x8, t);
    }
  }

  // ---- K/V staging: buffer loads straight into LDS.  Wave w's instruction u
  // fills the 1 KiB at chunk positions P = (w*NI + u)*64 + lane: row P/CPR,
  // physical column P%CPR.  The lane fetches the logical column that belongs
  // there (and, for K, the key the row holds: bits 2 and 3 of the row index
  // swapped, see k_lds_row).  Keys past the sequence end lie beyond the
  // resource's num_records and arrive as zeros.
  const int key_stride_b = p.hkv * D * 2;  // bytes between consecutive keys
  const char* kseq = (const char*)p.k + ((int64_t)si.k0 * p.hkv + g) * D * 2;
  const char* vseq = (const char*)p.v + ((int64_t)si.k0 * p.hkv + g) * D * 2;
  unsigned koff[NI], voff[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int P = (wave * NI + u) * 64 + lane;
    const int row = P / CPR, pc = P % CPR;
    koff[u] = (unsigned)(k_lds_row(row) * key_stride_b + ((pc ^ swz_k<D>(row)) * 16));
    voff[u] = (unsigned)(row * key_stride_b + ((pc ^ swz_v<D>(row)) * 16));
  }
  // LDS destination of this wave's first instruction, wave-uniform by construction
  const int wave_lds = __builtin_amdgcn_readfirstlane(wave * NI * 1024);
  auto stage = [&](const char* seq, const unsigned* off, char* dst, int n) __attribute__((always_inline)) {
    const int keys_left = si.sk - n * TN;  // > 0 for every staged block
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(seq + (int64_t)n * TN * key_stride_b), (short)0, keys_left * key_stride_b,
        kRsrcWord3);
#pragma unroll
    for (int u = 0; u < NI; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + wave_lds + u * 1024), 16,
                                               off[u], 0, 0, 0);
  };
  auto stage_k = [&](int n, int buf) __attribute__((always_inline)) { stage(kseq, koff, kbuf0 + buf * BUF, n); };
  auto stage_v = [&](int n, int buf) __attribute__((always_inline)) { stage(vseq, voff, vbuf0 + buf * BUF, n); };

  // K operand reads: lane (r32, hf) reads row 32t + r32, logical column
  // 2kc + hf of the K buffer.
  int ka[KC];
  {
    const int x = swz_k<D>(r32);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) ka[kc] = r32 * RB + (((2 * kc + hf) ^ x) * 16);
  }
  auto qk = [&](int buf, f32x16 (&s)[QG][2]) __attribute__((always_inline)) {
    const char* kb = kbuf0 + buf * BUF;
#pragma unroll
    for (int q = 0; q < QG; ++q)
#pragma unroll
      for (int t = 0; t < 2; ++t) s[q][t] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 a = *(const bf16x8*)(kb + 32 * t * RB + ka[kc]);
#pragma unroll
        for (int q = 0; q < QG; ++q)
          s[q][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[q][kc], s[q][t], 0, 0, 0);
      }
  };

  // Transposed V reads: lane = 16G + i reads 8 bytes of key row kb + i/4 at
  // dv columns 32dt + 16(G&1) + 4(i&3); after the transpose it holds
  // V[kb .. kb+3][32dt + 16(G&1) + i], its own A-operand column.  Rows kb are
  // multiples of 4, so the row's swizzle is swz_v(i/4) (D=128) and the
  // column part of the address depends only on dt.
  int va[DT];
  {
    const int tr_row = (lane & 15) >> 2;
    const int lc_lo = ((lane >> 4) & 1) * 2 + ((lane & 3) >> 1);  // 16-B column within 64 B
    const int half = (lane & 1) * 8;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int lc = 4 * t + lc_lo;
      // rows kb + tr_row with kb % 4 == 0: (kb + tr_row) & 3 = tr_row, and for
      // D=64 ((kb + tr_row) >> 1) & 1 = tr_row >> 1
      va[t] = (8 * hf + tr_row) * RB + ((lc ^ swz_v<D>(tr_row)) * 16) + half;
    }
  }

  // ---- running softmax state (per lane and group: one query, half of each key block)
  f32x16 oacc[QG][DT];
#pragma unroll
  for (int q = 0; q < QG; ++q)
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[q][t] = f32x16{};
  float m_run[QG], l_run[QG];
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    m_run[q] = -INFINITY;
    l_run[q] = 0.f;
  }

  // Pipeline: block n is consumed in iteration it = nblk-1-n; block j lives
  // in K/V buffer (nblk-1-j) & 1.  Iteration it computes S of block n-1 under
  // the softmax of block n, then O += P_n V_n, while the loads of K of block
  // n-2 and V of block n-1 fly into the buffers whose previous contents were
  // last read before this iteration's barrier; they are waited for before the
  // next barrier.  Iterations come in pairs (even it: buffer 0 is consumed,
  // odd: buffer 1), so the buffer addresses are constants and the two score
  // arrays swap roles instead of being copied.  The last iteration (n = 0)
  // also computes a score tile, from a stale K buffer, that nothing reads:
  // this keeps one copy of the loop body per buffer parity (a separate last
  // iteration made the register allocator spill).
  f32x16 s_a[QG][2], s_b[QG][2];
  stage_k(nblk - 1, 0);
  stage_v(nblk - 1, 0);
  if (nblk >= 2) stage_k(nblk - 2, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  qk(0, s_a);

  // One iteration.  sc: scores of block n; sn: receives those of block n-1
  // (unused when n = 0).  The four LDS regions are distinct within an
  // iteration (K and V being read, K and V being loaded); the __restrict__
  // qualifiers tell the compiler so, which keeps it from waiting for the
  // in-flight buffer->LDS loads before the transposed V reads.
  auto iteration = [&](const int it, f32x16 (&sc)[QG][2], f32x16 (&sn)[QG][2],
                       const char* __restrict__ kread, const char* __restrict__ vread,
                       char* __restrict__ kdst, char* __restrict__ vdst,
                       auto mask_tag) __attribute__((always_inline)) {
    const int n = nblk - 1 - it;
    __syncthreads();
    if (n >= 2) stage(kseq, koff, kdst, n - 2);
    if (n >= 1) stage(vseq, voff, vdst, n - 1);

    // mask: key of register r of sub-tile t is n*TN + 32t + 16(r/8) + 8hf + r%8
    if (decltype(mask_tag)::value) {
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        const int lim = CAUSAL ? min(si.sk - 1, qi[q] + diag) : si.sk - 1;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = n * TN + 32 * t + 16 * (r >> 3) + 8 * hf + (r & 7);
            if (key > lim) sc[q][t][r] = -INFINITY;
          }
      }
    }

    // P = exp2(c*S - c*m) against the running maximum, row sum, bf16 B
    // operands -- interleaved with the MFMAs of the next block's scores.  No
    // block maximum is taken first: the pass stands when every lane's share
    // of each row sum is at most kLazyBound (then no P exceeds the bound the
    // lazy rescale keeps); otherwise -- a maximum that grew, or a row with no
    // maximum yet, whose P are inf or NaN -- the block maximum is taken (in
    // lane, then across the two half-waves), O and l are rescaled to it where
    // it grew, and P is computed again.
    float rs[QG];
    bf16x8 pb[QG][4];
    auto expo = [&](const float (&ms)[QG], const int idx) __attribute__((always_inline)) {
      const int tt = idx >> 4, r = idx & 15;
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        const float pv = exp2_fast(__builtin_fmaf(sc[q][tt][r], c, -ms[q]));
        rs[q] = idx == 0 ? pv : rs[q] + pv;  // (0 + p is not folded)
        pb[q][2 * tt + (r >> 3)][r & 7] = (__bf16)pv;
      }
    };
    float ms[QG];
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      ms[q] = m_run[q] * c;
      rs[q] = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) sn[q][t] = f32x16{};
    }
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      const int kc = step >> 1, t = step & 1;
      if (kc < KC) {
        bf16x8 a = *(const bf16x8*)(kread + 32 * t * RB + ka[kc]);
#pragma unroll
        for (int q = 0; q < QG; ++q)
          sn[q][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[q][kc], sn[q][t], 0, 0, 0);
      }
      expo(ms, 2 * step);  // two of this lane's 32 scores per step and group
      expo(ms, 2 * step + 1);
    }
    bool redo = false;
#pragma unroll
    for (int q = 0; q < QG; ++q) redo = redo || !(rs[q] <= kLazyBound);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(redo) != 0, 0)) {
      float m_new[QG];
      bool grow = false;
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        m_new[q] = fmax_nan(m_run[q], halfwave_max(block_max(sc[q])));
        grow = grow || m_new[q] > m_run[q];
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        // With QG = 2 the O accumulators live in AGPRs and the scaling below
        // needs VGPR copies; redefining them here keeps the compiler from
        // hoisting those copies out of this rarely taken branch.
        if constexpr (QG == 2) {
#pragma unroll
          for (int q = 0; q < QG; ++q) pin_accumulators_agpr(oacc[q]);
        }
#pragma unroll
        for (int q = 0; q < QG; ++q) {
          // 0 when m_run = -inf < m_new; rows whose max is still -inf hold O =
          // 0 and l = 0 and keep them (their alpha would be exp2(NaN))
          const float alpha = m_new[q] == -INFINITY ? 1.f : exp2_fast((m_run[q] - m_new[q]) * c);
          m_run[q] = m_new[q];
          l_run[q] *= alpha;
#pragma unroll
          for (int t = 0; t < DT; ++t) oacc[q][t] *= alpha;
        }
      }
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        ms[q] = (m_run[q] == -INFINITY ? 0.f : m_run[q]) * c;
        rs[q] = 0.f;
      }
#pragma unroll
      for (int idx = 0; idx < 32; ++idx) expo(ms, idx);
    }
#pragma unroll
    for (int q = 0; q < QG; ++q) l_run[q] += rs[q];

    // O^T += V_n^T P^T
#pragma unroll
    for (int kc2 = 0; kc2 < 4; ++kc2) {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vread + 16 * kc2 * RB + va[t]));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vread + (16 * kc2 + 4) * RB + va[t]));
        bf16x4 lob = __builtin_bit_cast(bf16x4, lo), hib = __builtin_bit_cast(bf16x4, hi);
        bf16x8 a = {lob[0], lob[1], lob[2], lob[3], hib[0], hib[1], hib[2], hib[3]};
#pragma unroll
        for (int q = 0; q < QG; ++q)
          oacc[q][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[q][kc2], oacc[q][t], 0, 0, 0);
      }
    }
    if constexpr (QG == 1 && DT == 4) {
      // the transposed V reads kept four ahead of their MFMAs (left alone,
      // the compiler issues each MFMA's two reads right before it and waits
      // for them; measured 1 % slower on the packed varlen batch)
      sched_group(kSchedDsRead, 6);
#pragma unroll
      for (int i = 0; i < 13; ++i) {
        sched_group(kSchedMfma, 1);
        sched_group(kSchedDsRead, 2);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  // even iterations consume buffer 0 and load into K buffer 0 / V buffer 1;
  // odd iterations the other way round
  char* const k0b = kbuf0;
  char* const k1b = kbuf0 + BUF;
  char* const v0b = vbuf0;
  char* const v1b = vbuf0 + BUF;
  // Blocks are consumed from the last to the first, so the ones that need a
  // mask (past the end of the keys, or crossing the causal diagonal) come
  // first: block n needs one iff (n + 1) * TN > thr.  The masked iterations
  // (rounded up to an even count, so the unmasked loop starts on buffer 0)
  // run in a loop of their own; the main loop carries no mask code.
  const int thr = CAUSAL ? min(si.sk, m0 + diag + 1) : si.sk;
  const int n_plain = thr <= 0 ? 0 : min(nblk, thr / TN);  // blocks 0 .. n_plain-1 need no mask
  const int it_mask_end = min(nblk, (nblk - n_plain + 1) & ~1);
  int it = 0;
  for (; it < it_mask_end; it += 2) {
    iteration(it, s_a, s_b, k1b, v0b, k0b, v1b, BoolTag<true>{});
    if (it + 1 == nblk) {
      it = nblk;
      break;
    }
    iteration(it + 1, s_b, s_a, k0b, v1b, k1b, v0b, BoolTag<true>{});
  }
  for (; it < nblk; it += 2) {
    iteration(it, s_a, s_b, k1b, v0b, k0b, v1b, BoolTag<false>{});
    if (it + 1 == nblk) break;
    iteration(it + 1, s_b, s_a, k0b, v1b, k1b, v0b, BoolTag<false>{});
  }

  // ---- epilogue: normalise, O (bf16) and LSE (natural log)
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    if constexpr (QG == 1) pin_accumulators(oacc[q]);
    else pin_accumulators_agpr(oacc[q]);
  }
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    const float l_tot = halfwave_sum(l_run[q]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    store_o_rows<DT>(oacc[q], inv, O + orow[q], hf, qvalid[q]);
    if (qvalid[q] && hf == 0)
      p.lse[lse_idx[q]] = l_tot > 0.f ? (m_run[q] * c + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong schedule (bf16).  A workgroup of 8 waves (two per SIMD) takes one
// 128-row query tile of TWO query heads that share a KV head -- or, with an
// odd number of query heads per KV head (1 for MHA), two adjacent 128-row
// tiles of one head -- so both halves walk the same key blocks out of one K/V
// staging.
// Waves 0-3 (group A, first head) and 4-7 (group B, second head) alternate
// between a GEMM slot -- the QK^T of the next block and the P V of the current
// one, with all their LDS operand reads -- and a softmax slot (VALU and the
// transcendental unit only), offset by one slot: while one wave of a SIMD
// keeps the matrix core busy, the other exponentiates.  Each step starts at
// a workgroup barrier; within it the groups run their two phases back to back
// in opposite order.  Step k (k = 0 .. N, N key blocks, block N-1-k is the
// one whose scores step k computes):
//   slot 2k:   A: GEMM(k)            B: softmax of block N-k (k >= 1)
//   slot 2k+1: A: softmax of N-1-k   B: GEMM(k)
// GEMM(k) = S <- K_{N-1-k} Q^T (k < N) and O += V_{N-k}^T P^T (k >= 1).  K_j
// lives in K buffer (N-1-j) & 1 and V_j in V buffer (N-1-j) & 1; at the start
// of slot 2k (k >= 1) all eight waves load K_{N-2-k} and V_{N-1-k}, two slots
// before their first use, into the buffers whose last readers finished in
// slot 2k-1; the prologue loads step 0's share (K_{N-1}, K_{N-2}, V_{N-1}).
// XQ > 0 puts every XQ-th exponential on the FMA polynomial (exp2 offload).
#ifndef PP_LEAD
#define PP_LEAD 4
#endif
// One work item of the ping-pong schedule, for the kernel that gives each
// workgroup one item (PERSIST false) and for the persistent kernel below.
// smem: 4 * BUF bytes of K/V stages, and with PERSIST a Q stage of 32 rows per
// wave after them.  wid_in: the item; next_wid (PERSIST): the item this
// workgroup takes next, whose query rows are prefetched into the Q stage
// during this one (-1: none); q_in_lds: this item's rows were prefetched so.
// Returns whether it prefetched.
template <int D, bool CAUSAL, int XQ, bool PERSIST>
__device__ __forceinline__ bool pp_item(const Params& p, char* const smem, const int wid_in,
                                        const int next_wid, const bool q_in_lds) {
  constexpr int TM = kTileM, TN = kTileN;
  constexpr int RB = D * 2;                  // bytes per K/V row in LDS
  constexpr int BUF = TN * RB;               // bytes per K or V block buffer
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NW = 8;                      // waves per workgroup
  constexpr int NI = TN * CPR / (64 * NW);   // direct-load instructions per wave per block
  constexpr int KC = D / 16;                 // k-chunks of the QK^T product
  constexpr int DT = D / 32;                 // 32-wide output tiles of O^T
  static_assert(NI >= 1, "each wave issues at least one load per block");
  char* const kbuf0 = smem;
  char* const vbuf0 = smem + 2 * BUF;

  // Persistent: the item id is wave-uniform by construction and said so, and
  // the thread index passes an empty asm per item, so that nothing derived
  // from it is hoisted out of the item loop (where it would hold registers
  // through every step of every item).
  const int wid = PERSIST ? __builtin_amdgcn_readfirstlane(wid_in) : wid_in;
  int tid = threadIdx.x;
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int wave = tid >> 6;
  const int grp = wave >> 2;  // 0: group A, 1: group B
  // 32-row slice of the tile; group B takes the slices in reverse order, so
  // that each SIMD holds a low and a high slice (waves w and w + 4 share one)
  // and the causal diagonal's fully masked blocks, which the low slices skip,
  // lighten every SIMD alike
  const int wv = grp == 0 ? (wave & 3) : 3 - (wave & 3);
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  // ---- work item: the XCD deal of the 4-wave kernel, with pairs of query
  // heads in place of query heads.  With an odd number of query heads per
  // KV head (1 for MHA) the two groups take two adjacent 128-row query tiles
  // of one head instead (p.m_tiles then counts tile pairs): they still read
  // the same K/V blocks, those of the upper tile, whose extra causal blocks
  // are fully masked for the lower one.
  const bool mpair = p.group & 1;
  struct Item {
    int g, head, m0_wg, m0;  // KV head, this group's query head, first rows
    SeqInfo si;
  };
  // false for the padding of the last round and for a tile past its
  // sequence's end (uniform over the workgroup, decided before any barrier)
  auto decode = [&](const int id, Item& it) __attribute__((always_inline)) {
    const int hpairs = mpair ? p.group : p.group >> 1;  // slots per (tile, KV head)
    ItemIdx itx;
    if (!item_index(p, (unsigned)id, hpairs, itx)) return false;
    const int pair = itx.pair, mrev = itx.mrev;
    const int b = pair / p.hkv;
    it.g = pair - b * p.hkv;
    it.head = mpair ? it.g * p.group + itx.hsub : it.g * p.group + 2 * itx.hsub + grp;
    const int mblk = CAUSAL ? (p.m_tiles - 1 - mrev) : mrev;
    it.si = seq_info(p, b);
    if constexpr (PERSIST) {
      it.si.q0 = __builtin_amdgcn_readfirstlane(it.si.q0);
      it.si.sq = __builtin_amdgcn_readfirstlane(it.si.sq);
      it.si.k0 = __builtin_amdgcn_readfirstlane(it.si.k0);
      it.si.sk = __builtin_amdgcn_readfirstlane(it.si.sk);
      it.si.total_q = __builtin_amdgcn_readfirstlane(it.si.total_q);
    }
    it.m0_wg = mpair ? 2 * mblk * TM : mblk * TM;  // the workgroup's first row
    it.m0 = mpair ? it.m0_wg + grp * TM : it.m0_wg;  // this group's first row
    return it.m0_wg < it.si.sq;
  };
  Item cur;
  if (!decode(wid, cur)) return false;
  const int g = cur.g, head = cur.head, m0_wg = cur.m0_wg, m0 = cur.m0;
  const SeqInfo si = cur.si;
  const int m0_top = mpair ? m0_wg + TM : m0_wg;       // the upper group's first row
  const int qi = m0 + wv * 32 + r32;
  const bool qvalid = qi < si.sq;

  const __bf16* __restrict__ Q = (const __bf16*)p.q;
  __bf16* __restrict__ O = (__bf16*)p.o;
  const float c = p.scale_log2;

  const int diag = si.sk - si.sq;  // bottom-right alignment offset
  int kend = si.sk;
  if (CAUSAL) kend = min(kend, m0_top + TM + diag);
  const int N = kend > 0 ? (kend + TN - 1) / TN : 0;

  auto orow = [&]() __attribute__((always_inline)) {
    return ((int64_t)(si.q0 + qi) * p.hq + head) * D;
  };
  auto lse_idx = [&]() __attribute__((always_inline)) {
    return (int64_t)head * si.total_q + si.q0 + qi;
  };

  if (N == 0) {  // store_zero
    if (qvalid) {
      for (int e = hf * 4; e < D; e += 8) *(u32x2*)(O + orow() + e) = u32x2{0u, 0u};
      if (hf == 0) p.lse[lse_idx()] = -INFINITY;
    }
    return false;
  }

  bf16x8 qf[KC];
  if (!PERSIST || !q_in_lds) {
    const __bf16* qp = Q + orow() + 8 * hf;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 t = qvalid ? *(const u32x4*)(qp + 16 * kc) : u32x4{0u, 0u, 0u, 0u};
      qf[kc] = __builtin_bit_cast(bf16x8, t);
    }
  }

  // ---- K/V staging (as the 4-wave kernel; eight waves share each block)
  const int key_stride_b = p.hkv * D * 2;
  const char* kseq = (const char*)p.k + ((int64_t)si.k0 * p.hkv + g) * D * 2;
  const char* vseq = (const char*)p.v + ((int64_t)si.k0 * p.hkv + g) * D * 2;
  unsigned koff[NI], voff[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int P = (wave * NI + u) * 64 + lane;
    const int row = P / CPR, pc = P % CPR;
    koff[u] = (unsigned)(k_lds_row(row) * key_stride_b + ((pc ^ swz_k<D>(row)) * 16));
    voff[u] = (unsigned)(row * key_stride_b + ((pc ^ swz_v<D>(row)) * 16));
  }
  const int wave_lds = __builtin_amdgcn_readfirstlane(wave * NI * 1024);
  auto stage = [&](const char* seq, const unsigned* off, char* dst, int n) __attribute__((always_inline)) {
    const int keys_left = si.sk - n * TN;  // > 0 for every staged block
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(seq + (int64_t)n * TN * key_stride_b), (short)0, keys_left * key_stride_b,
        kRsrcWord3);
#pragma unroll
    for (int u = 0; u < NI; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + wave_lds + u * 1024), 16,
                                               off[u], 0, 0, 0);
  };

  int ka[KC];
  {
    const int x = swz_k<D>(r32);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) ka[kc] = r32 * RB + (((2 * kc + hf) ^ x) * 16);
  }
  // Persistent: this wave's Q stage (its 32 query rows of the next item), 16-byte
  // chunk c of row r at position c ^ swz_k(r) -- the K layout, so the K operand
  // offsets address the B operand fragments
  char* const qwave = smem + 4 * BUF + __builtin_amdgcn_readfirstlane(wave * 32 * RB);
  if constexpr (PERSIST) {
    if (q_in_lds) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) qf[kc] = *(const bf16x8*)(qwave + ka[kc]);
    }
  }
  // The next item's rows are loaded into the Q stage in step kq, after that
  // step's K/V loads; the barrier of step kq + 1 then waits for all but
  // these NQ loads, and the epilogue for them before its stores.
  constexpr int NQ = 32 * CPR / 64;  // 16-byte loads per lane
  const int kq = N > 3 ? N - 2 : 1;
  bool pf_done = false;
  auto prefetch_q = [&]() __attribute__((always_inline)) {
    if constexpr (PERSIST) {
      Item nx;
      const int nwid = __builtin_amdgcn_readfirstlane(next_wid);
      if (nwid < 0 || !decode(nwid, nx)) return;
      pf_done = true;
      const int r0 = nx.m0 + wv * 32;
      const int rows = min(max(nx.si.sq - r0, 0), 32);  // rows past the end arrive as zeros
      const int rstride = p.hq * D * 2;
      const char* base = (const char*)p.q + ((int64_t)(nx.si.q0 + r0) * p.hq + nx.head) * D * 2;
      __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows * rstride, kRsrcWord3);
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int P = u * 64 + lane;
        const int row = P / CPR, pos = P % CPR;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void*)(qwave + u * 1024), 16,
            (unsigned)(row * rstride + ((pos ^ swz_k<D>(row)) * 16)), 0, 0, 0);
      }
    }
  };
  int va[DT];
  {
    const int tr_row = (lane & 15) >> 2;
    const int lc_lo = ((lane >> 4) & 1) * 2 + ((lane & 3) >> 1);
    const int half = (lane & 1) * 8;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int lc = 4 * t + lc_lo;
      va[t] = (8 * hf + tr_row) * RB + ((lc ^ swz_v<D>(tr_row)) * 16) + half;
    }
  }

  // ---- per-wave state: one score tile, one P tile, O, running max and sum
  f32x16 sc[2];
  bf16x8 pb[4];
  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Causal: the top ktop blocks hold no admissible key for any row of this
  // wave (its last row sees keys up to m0 + 32 wv + 31 + diag); they are
  // skipped -- scores, softmax and P V -- in the first steps, which run with
  // these per-wave checks (ks of them, bounded by the workgroup's lowest row).
  int ktop = 0, ks = 0;
  if (CAUSAL) {
    const int last = m0 + wv * 32 + 31 + diag;
    ktop = last < 0 ? N : max(0, N - 1 - last / TN);
    const int wg_last = m0_wg + 31 + diag;
    ks = wg_last < 0 ? N + 1 : min(N + 1, max(0, N - 1 - wg_last / TN) + 1);
  }
  const int thr = CAUSAL ? min(si.sk, m0 + diag + 1) : si.sk;
  const int n_plain = thr <= 0 ? 0 : min(N, thr / TN);  // blocks below n_plain need no mask

  // softmax slot for block j: mask, running max, lazy rescale, P and row sum
  auto softmax = [&](const int j) __attribute__((always_inline)) {
    if (j >= n_plain) {
      const int lim = CAUSAL ? min(si.sk - 1, qi + diag) : si.sk - 1;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * TN + 32 * t + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (key > lim) sc[t][r] = -INFINITY;
        }
    }
    // P is first taken against the running maximum without the block's own
    // maximum.  The pass stands when every lane's share of the row sum is at
    // most kLazyBound: then no P exceeds it, the bound the lazy rescale keeps.
    // Otherwise (a maximum that grew, a row with no maximum yet: its P are
    // inf or NaN) the block maximum is taken, O and l are rescaled to it if
    // it grew, and P is computed again.  Saves the max reduction (a sixth of
    // the softmax's instructions) on nearly every block.
    auto expo = [&](const float ms) __attribute__((always_inline)) {
      float rs = 0.f;
#pragma unroll
      for (int idx = 0; idx < 32; ++idx) {
        const int tt = idx >> 4, r = idx & 15;
        // XQ > 0: every XQ-th exponential on the FMA polynomial (exp2 offload)
        const float x = __builtin_fmaf(sc[tt][r], c, -ms);
        const float pv = (XQ > 0 && idx % XQ == XQ - 1) ? exp2_poly(x) : exp2_fast(x);
        rs = idx == 0 ? pv : rs + pv;  // (0 + p is not folded)
        pb[2 * tt + (r >> 3)][r & 7] = (__bf16)pv;
      }
      return rs;
    };
    float rs = expo(m_run * c);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(rs <= kLazyBound)) != 0, 0)) {
      const float m_new = fmax_nan(m_run, halfwave_max(block_max(sc)));
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        const float alpha = m_new == -INFINITY ? 1.f : exp2_fast((m_run - m_new) * c);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
      }
      rs = expo((m_run == -INFINITY ? 0.f : m_run) * c);
    }
    l_run += rs;
  };

  // GEMM slot: QK of the next block and P V of the current one, interleaved
  auto gemm = [&](const char* __restrict__ kread, const char* __restrict__ vread, auto qk_tag,
                  auto pv_tag) __attribute__((always_inline)) {
    constexpr bool DO_QK = decltype(qk_tag)::value;
    constexpr bool DO_PV = decltype(pv_tag)::value;
    if (DO_QK) {
#pragma unroll
      for (int t = 0; t < 2; ++t) sc[t] = f32x16{};
    }
    constexpr int STEPS = 2 * KC > 4 * DT ? 2 * KC : 4 * DT;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      if (DO_QK && st < 2 * KC) {
        const int kc = st >> 1, t = st & 1;
        bf16x8 a = *(const bf16x8*)(kread + 32 * t * RB + ka[kc]);
        sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], sc[t], 0, 0, 0);
      }
      if (DO_PV && st < 4 * DT) {
        const int kc2 = st / DT, t = st % DT;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vread + 16 * kc2 * RB + va[t]));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vread + (16 * kc2 + 4) * RB + va[t]));
        bf16x4 lob = __builtin_bit_cast(bf16x4, lo), hib = __builtin_bit_cast(bf16x4, hi);
        bf16x8 a = {lob[0], lob[1], lob[2], lob[3], hib[0], hib[1], hib[2], hib[3]};
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc2], oacc[t], 0, 0, 0);
      }
    }
    if (DO_QK && DO_PV) {
      // Only this wave of the SIMD issues MFMAs during the slot, so nothing
      // else hides LDS latency.  The slot reads 1.5 operands per MFMA (a K
      // row block for QK^T, two transposed V reads for P V): PP_LEAD reads go
      // first, then each pair of MFMAs is followed by three reads, so the
      // reads stay PP_LEAD ahead to the end of the slot.  (A lead that is
      // large up front and shrinks by half a read per MFMA stalls at both
      // ends: the first MFMA waits for all but 15 of the reads issued before
      // it -- the LDS counter's limit -- and the last ones for reads just
      // issued; measured 0.6-1.4 % slower.)
      sched_group(kSchedDsRead, PP_LEAD);
#pragma unroll
      for (int i = 0; i < (3 * STEPS - PP_LEAD) / 3; ++i) {
        sched_group(kSchedMfma, 1);
        sched_group(kSchedDsRead, 2);
        sched_group(kSchedMfma, 1);
        sched_group(kSchedDsRead, 1);
      }
    }
  };

  // One step: the full barrier (the loads issued two slots ago are complete
  // and visible, the buffers read in slot 2k-1 are free), this step's loads,
  // the two slots.  The barrier between the slots only orders the phases.
  // The four LDS regions are distinct within a step; __restrict__ says so,
  // which keeps the compiler from waiting for the loads before LDS reads.
  auto step = [&](const int k, const char* __restrict__ kread, const char* __restrict__ vread,
                  char* __restrict__ kdst, char* __restrict__ vdst, auto qk_tag, auto pv_tag,
                  auto skip_tag) __attribute__((always_inline)) {
    // Each wave's own direct-to-LDS loads must be complete before the barrier
    // for the other waves to read them.  The wait is written out: the
    // barrier's fence does not oblige the compiler to wait for loads, and in
    // some code shapes it does not.
    if (PERSIST && pf_done && k == kq + 1) {
      if constexpr (NQ == 8)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    // Group A issues its share of the step's loads at the step start, group B
    // after its softmax phase, so that B's softmax -- running beside A's
    // GEMM phase -- starts at once (measured +0.8 % on the bench workload,
    // +0.6 to +1.5 % elsewhere; A's share after its GEMM phase: -0.6 %)
    auto loads = [&]() __attribute__((always_inline)) {
      if (k >= 1) {  // step 0's loads are part of the prologue
        if (N - 2 - k >= 0) stage(kseq, koff, kdst, N - 2 - k);
        if (N - 1 - k >= 0) stage(vseq, voff, vdst, N - 1 - k);
        if (PERSIST && k == kq) prefetch_q();
      }
    };
    if (grp == 0) loads();
    // The two phases follow each other without a barrier (one between them
    // would publish nothing): the step's full barrier starts the groups in
    // opposite phases, a group that finishes its first phase early starts its
    // second at once, and the GEMM phase runs at raised wave priority so that
    // the SIMD's other wave, in its softmax phase, yields the issue slots the
    // matrix instructions and their LDS reads need.  The s_setprio
    // instructions also keep the compiler from mixing the two phases' code.
    // Measured 1.6 % faster than a barrier between the phases.
    // with skips (first steps, causal): block N-1-k has no admissible key for
    // this wave when k < ktop, block N-k when k <= ktop
    const bool chk = decltype(skip_tag)::value;
    const bool sk_q = chk && k < ktop, sk_p = chk && k <= ktop;
    auto gemm_sk = [&]() __attribute__((always_inline)) {
      constexpr bool Q = decltype(qk_tag)::value, PV = decltype(pv_tag)::value;
      if (!chk) {
        gemm(kread, vread, qk_tag, pv_tag);
      } else if (Q && PV) {
        if (!sk_q && !sk_p) gemm(kread, vread, BoolTag<true>{}, BoolTag<true>{});
        else if (!sk_q) gemm(kread, vread, BoolTag<true>{}, BoolTag<false>{});
        else if (!sk_p) gemm(kread, vread, BoolTag<false>{}, BoolTag<true>{});
      } else if (Q) {
        if (!sk_q) gemm(kread, vread, BoolTag<true>{}, BoolTag<false>{});
      } else if (PV) {
        if (!sk_p) gemm(kread, vread, BoolTag<false>{}, BoolTag<true>{});
      }
    };
    if (grp == 0) {
      __builtin_amdgcn_s_setprio(1);
      gemm_sk();
      __builtin_amdgcn_s_setprio(0);
      if (k < N && !sk_q) softmax(N - 1 - k);
    } else {
      if (k >= 1 && !sk_p) softmax(N - k);
      loads();
      __builtin_amdgcn_s_setprio(1);
      gemm_sk();
      __builtin_amdgcn_s_setprio(0);
    }
  };
  auto bufs = [&](const int k, const char*& kr, const char*& vr, char*& kd, char*& vd)
      __attribute__((always_inline)) {
    const int par = k & 1;
    kr = kbuf0 + par * BUF;
    kd = kbuf0 + (par ^ 1) * BUF;
    vr = vbuf0 + (par ^ 1) * BUF;
    vd = vbuf0 + par * BUF;
  };

  // the prologue loads what steps 0 and 1 read: K_{N-1} (buffer 0), K_{N-2}
  // (buffer 1) and V_{N-1} (V buffer 0), so the short step 0 leaves no load
  // in flight for step 1's barrier to wait out
  stage(kseq, koff, kbuf0, N - 1);
  if (N >= 2) stage(kseq, koff, kbuf0 + BUF, N - 2);
  stage(vseq, voff, vbuf0, N - 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  {
    const char *kr, *vr;
    char *kd, *vd;
    bufs(0, kr, vr, kd, vd);
    if (CAUSAL && ks > 0)
      step(0, kr, vr, kd, vd, BoolTag<true>{}, BoolTag<false>{}, BoolTag<true>{});
    else
      step(0, kr, vr, kd, vd, BoolTag<true>{}, BoolTag<false>{}, BoolTag<false>{});
    int k = 1;
    if (CAUSAL) {
      for (; k < min(N, ks); ++k) {
        bufs(k, kr, vr, kd, vd);
        step(k, kr, vr, kd, vd, BoolTag<true>{}, BoolTag<true>{}, BoolTag<true>{});
      }
    }
    // pairs of steps with the buffers as constants (even k: K buffer 0 and
    // V buffer 1 are read), so that the buffer offsets are immediates of the
    // LDS reads instead of a vector add per address (measured +0.7 %)
    if (k < N && (k & 1)) {
      bufs(k, kr, vr, kd, vd);
      step(k, kr, vr, kd, vd, BoolTag<true>{}, BoolTag<true>{}, BoolTag<false>{});
      ++k;
    }
    for (; k + 1 < N; k += 2) {
      step(k, kbuf0, vbuf0 + BUF, kbuf0 + BUF, vbuf0, BoolTag<true>{}, BoolTag<true>{}, BoolTag<false>{});
      step(k + 1, kbuf0 + BUF, vbuf0, kbuf0, vbuf0 + BUF, BoolTag<true>{}, BoolTag<true>{},
           BoolTag<false>{});
    }
    if (k < N) {
      bufs(k, kr, vr, kd, vd);
      step(k, kr, vr, kd, vd, BoolTag<true>{}, BoolTag<true>{}, BoolTag<false>{});
      ++k;
    }
    bufs(N, kr, vr, kd, vd);
    if (CAUSAL && ks > N)
      step(N, kr, vr, kd, vd, BoolTag<false>{}, BoolTag<true>{}, BoolTag<true>{});
    else
      step(N, kr, vr, kd, vd, BoolTag<false>{}, BoolTag<true>{}, BoolTag<false>{});
  }

  // ---- epilogue
  // the next item's query rows are in this wave's Q stage before the stores
  // (later loads would otherwise wait behind them)
  if (PERSIST && pf_done) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  pin_accumulators(oacc);
  const float l_tot = halfwave_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  store_o_rows<DT>(oacc, inv, O + orow(), hf, qvalid);
  if (qvalid && hf == 0)
    p.lse[lse_idx()] = l_tot > 0.f ? (m_run * c + __log2f(l_tot)) * kLn2 : -INFINITY;
  return pf_done;
}

template <int D, bool CAUSAL, int XQ>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_pp_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileN * D * 2];
  pp_item<D, CAUSAL, XQ, false>(p, smem, blockIdx.x, -1, false);
}

// Persistent ping-pong (schedule 5, forced only): one resident workgroup per
// CU walking the items of its XCD (item = kXcds * slot + xcd, the order of the
// one-item kernel: heaviest tiles first, neighbouring slots on one KV head).
// The gridDim.x / kXcds workgroups of an XCD take its slots in windows of
// twice their number, zig-zag within each window (workgroup w: slots w and
// 2G - 1 - w), which balances the causal tiles' work while all of them stay
// on neighbouring slots, and each prefetches the query rows of its next item
// before the epilogue of the current one ([FWD-PASS] producer loop: the next
// work tile is fetched before the epilogue).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_pp_persist_kernel(Params p, int num_items) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileN * D * 2 + 8 * 32 * D * 2];
  const int G = gridDim.x / kXcds, w = blockIdx.x / kXcds, x = blockIdx.x % kXcds;
  const int slots = num_items / kXcds;
  auto slot_of = [&](const int r) { return 2 * G * (r >> 1) + ((r & 1) ? 2 * G - 1 - w : w); };
  bool q_in_lds = false;
  for (int r = 0; 2 * G * (r >> 1) < slots; ++r) {
    const int slot = slot_of(r), nslot = slot_of(r + 1);
    if (r > 0) __syncthreads();  // the previous item's readers are done with the stages
    q_in_lds = slot < slots && pp_item<D, CAUSAL, 0, true>(p, smem, slot * kXcds + x,
                                                            nslot < slots ? nslot * kXcds + x : -1,
                                                            q_in_lds);
  }
}

// ---------------------------------------------------------------------------
// Decode schedule (bf16; heads_q / heads_kv * seqlen_q <= 32).  Every query
// row of one KV head's group -- the (query head, row) pairs -- fits the 32
// columns of one MFMA tile, so a workgroup takes one (sequence, KV head) whole
// and its four waves split the key range instead: wave w takes the 32-key
// blocks w, w+4, w+8, ... Each wave streams its K and V blocks through a
// private LDS ring (laid out as the other kernels lay out theirs), one block
// ahead, so the loop has no barrier; K staged in LDS rather than loaded into
// registers in operand order keeps the loads at 16 lanes per row (a quarter
// of the cache-line requests), which measured 8-33 % faster.  Each wave keeps the running
// maximum, sum and O of the online softmax over its own blocks ([FWD-PASS]
// consumer loop); the four partial states merge at the end through LDS with
// the same rescaling the recurrence uses between blocks: with M the largest
// partial maximum, O = sum_w 2^{c(m_w - M)} O_w / sum_w 2^{c(m_w - M)} l_w.
// The work per key is small (at most 32 useful columns), so the kernel is
// bound by streaming K and V from HBM.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_bf16_decode_kernel(Params p) {
  constexpr int TK = 32;                 // keys per block
  constexpr int RB = D * 2;              // bytes per K/V row
  constexpr int VBUF = TK * RB;          // one V block in LDS
  constexpr int NSTG = kDecodeSlots;     // K and V ring slots per wave
  constexpr int DEPTH = NSTG - 1;        // blocks loading while one is in use
  constexpr int KC = D / 16;             // k-chunks of QK^T
  constexpr int DT = D / 32;             // 32-dim tiles of O^T
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int NWV = kDecodeWaves;      // waves
  static_assert(NWV >= 1 && NWV <= 4,
                "one wave per SIMD: the kernel holds the full 512-register file");
  constexpr int VI = TK * CPR / 64;      // direct-load instructions per V block
  constexpr int BLK_LOADS = 2 * VI;      // memory instructions per block and wave
  static_assert(DEPTH * BLK_LOADS <= 63, "vmcnt counts up to 63");
  constexpr int WAVE_LDS = 2 * NSTG * VBUF;
  static_assert(NWV * (DT * 4096 + 512) <= NWV * WAVE_LDS, "the merge area fits the rings");
  __shared__ __attribute__((aligned(1024))) char smem[NWV * WAVE_LDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hf = lane >> 5;
  char* const ring = smem + wave * WAVE_LDS;   // V slots, then K slots
  char* const kring = ring + NSTG * VBUF;

  const int b = blockIdx.x / p.hkv;
  const int g = blockIdx.x - b * p.hkv;
  const SeqInfo si = seq_info(p, b);
  if (si.sq <= 0) return;  // uniform: no query rows
  // this lane's column: query head g*group + hloc, query row qrow
  const int hloc = r32 / si.sq;
  const int qrow = r32 - hloc * si.sq;
  const bool cvalid = hloc < p.group;
  const int head = g * p.group + hloc;
  const float c = p.scale_log2;
  const int diag = si.sk - si.sq;  // bottom-right alignment offset
  // the last query row sees every key (bottom-right alignment), so all
  // ceil(sk / TK) blocks are read
  const int nb = si.sk > 0 ? (si.sk + TK - 1) / TK : 0;
  const int nmine = nb > wave ? (nb - wave + NWV - 1) / NWV : 0;
  const int lim = CAUSAL ? min(si.sk - 1, qrow + diag) : si.sk - 1;  // last key of this column

  // Q^T as the B operand: lane (column, hf) holds dims 16kc + 8hf .. +7
  bf16x8 qf[KC];
  {
    const __bf16* qp = (const __bf16*)p.q + ((int64_t)(si.q0 + qrow) * p.hq + head) * D + 8 * hf;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 t = cvalid ? *(const u32x4*)(qp + 16 * kc) : u32x4{0u, 0u, 0u, 0u};
      qf[kc] = __builtin_bit_cast(bf16x8, t);
    }
  }

  const int key_stride_b = p.hkv * D * 2;
  const char* kseq = (const char*)p.k + ((int64_t)si.k0 * p.hkv + g) * D * 2;
  const char* vseq = (const char*)p.v + ((int64_t)si.k0 * p.hkv + g) * D * 2;
  unsigned voff[VI], koff[VI];
#pragma unroll
  for (int u = 0; u < VI; ++u) {
    const int P = u * 64 + lane;
    const int row = P / CPR, pc = P % CPR;
    voff[u] = (unsigned)(row * key_stride_b + ((pc ^ swz_v<D>(row)) * 16));
    koff[u] = (unsigned)(k_lds_row(row) * key_stride_b + ((pc ^ swz_k<D>(row)) * 16));
  }
  int ka[KC];
  {
    const int x = swz_k<D>(r32);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) ka[kc] = r32 * RB + (((2 * kc + hf) ^ x) * 16);
  }
  int va[DT];
  {
    const int tr_row = (lane & 15) >> 2;
    const int lc_lo = ((lane >> 4) & 1) * 2 + ((lane & 3) >> 1);
    const int half = (lane & 1) * 8;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int lc = 4 * t + lc_lo;
      va[t] = (8 * hf + tr_row) * RB + ((lc ^ swz_v<D>(tr_row)) * 16) + half;
    }
  }

  // Block i of this wave (key block j = wave + NWV*i) into ring slot i % NSTG.
  // Keys at or past sk lie beyond the resources' num_records and arrive as
  // zeros.  (Device pass only: the host pass drops the kernel's launch stub
  // when this lambda calls the buffer-load builtins.)
  auto issue = [&](const int i) __attribute__((always_inline)) {
#if __HIP_DEVICE_COMPILE__
    const int j = wave + NWV * i;
    const int keys_left = si.sk - j * TK;  // > 0: j < nb
    const char* kb = kseq + (int64_t)j * TK * key_stride_b;
    const char* vb = vseq + (int64_t)j * TK * key_stride_b;
    __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, keys_left * key_stride_b, kRsrcWord3);
    __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, keys_left * key_stride_b, kRsrcWord3);
    char* dst = ring + __builtin_amdgcn_readfirstlane((i % NSTG) * VBUF);
#pragma unroll
    for (int u = 0; u < VI; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst + NSTG * VBUF + u * 1024), 16,
                                               koff[u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < VI; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst + u * 1024), 16, voff[u], 0,
                                               0, 0);
#endif
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    if (i < nmine) issue(i);

  // Blocks in groups of NSTG so that every slot offset is a constant: block
  // bb uses slot s = bb % NSTG; block bb + DEPTH goes to the slot that block
  // bb - 1 released.
  for (int i = 0; i < nmine; i += NSTG) {
#pragma unroll
    for (int s = 0; s < NSTG; ++s) {
      const int bb = i + s;
      if (bb >= nmine) break;
      if (bb + DEPTH < nmine) issue(bb + DEPTH);
      // Block bb's loads are complete once at most the blocks issued after
      // it are outstanding (its V copy lands in LDS by the same count).  The
      // asm keeps every memory access on its side of the wait.
      const int newer = min(DEPTH, nmine - 1 - bb);
      if (DEPTH >= 3 && newer >= 3)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * BLK_LOADS) : "memory");
      else if (DEPTH >= 2 && newer == 2)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * BLK_LOADS) : "memory");
      else if (newer == 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(BLK_LOADS) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const char* vslot = ring + s * VBUF;

      // S^T = K Q^T: two accumulators over alternating k-chunks
      f32x16 sa = f32x16{}, sb = f32x16{};
      const char* kslot = kring + s * VBUF;
#pragma unroll
      for (int kc = 0; kc < KC; kc += 2) {
        const bf16x8 a0 = *(const bf16x8*)(kslot + ka[kc]);
        const bf16x8 a1 = *(const bf16x8*)(kslot + ka[kc + 1]);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kc], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kc + 1], sb, 0, 0, 0);
      }
      f32x16 sc = sa + sb;
      // register r of half hf holds key j*TK + 16(r>>3) + 8hf + (r&7)
      const int j = wave + NWV * bb;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j * TK + 16 * (r >> 3) + 8 * hf + (r & 7);
        if (key > lim || !cvalid) sc[r] = -INFINITY;
      }
      float mx = fmax_nan(sc[0], sc[1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmax_nan(fmax_nan(mx, sc[r]), sc[r + 1]);
      const float m_new = fmax_nan(m_run, halfwave_max(mx));
      if (__builtin_amdgcn_ballot_w64((m_new - m_run) * c > kLazy) != 0) {
        const float alpha = m_new == -INFINITY ? 1.f : exp2_fast((m_run - m_new) * c);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
      }
      const float ms = (m_run == -INFINITY ? 0.f : m_run) * c;
      bf16x8 pb[2];
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_fast(__builtin_fmaf(sc[r], c, -ms));
        rs = r == 0 ? pv : rs + pv;  // (0 + p is not folded)
        pb[r >> 3][r & 7] = (__bf16)pv;
      }
      l_run += rs;
      // O^T += V^T P^T over the block's two 16-key chunks
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2)
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vslot + 16 * kc2 * RB + va[t]));
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vslot + (16 * kc2 + 4) * RB + va[t]));
          bf16x4 lob = __builtin_bit_cast(bf16x4, lo), hib = __builtin_bit_cast(bf16x4, hi);
          bf16x8 a = {lob[0], lob[1], lob[2], lob[3], hib[0], hib[1], hib[2], hib[3]};
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc2], oacc[t], 0, 0, 0);
        }
    }
  }

  // ---- merge the four waves' partial states through LDS (the rings are free
  // once every wave is past its loop)
  pin_accumulators(oacc);
  const float l_tot = halfwave_sum(l_run);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  char* const mine = smem + wave * (DT * 4096 + 512);
#pragma unroll
  for (int t = 0; t < DT; ++t) *(f32x16*)(mine + t * 4096 + lane * 64) = oacc[t];
  *(float2*)(mine + DT * 4096 + lane * 8) = float2{m_run, l_tot};
  __syncthreads();
  float mw[NWV], lw[NWV];
  float mmax = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const float2 ml = *(const float2*)(smem + w * (DT * 4096 + 512) + DT * 4096 + lane * 8);
    mw[w] = ml.x;
    lw[w] = ml.y;
    mmax = fmax_nan(mmax, ml.x);
  }
  float wt[NWV], L = 0.f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    wt[w] = mmax == -INFINITY ? 0.f : exp2_fast((mw[w] - mmax) * c);
    L += wt[w] * lw[w];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  __bf16* orow = (__bf16*)p.o + ((int64_t)(si.q0 + qrow) * p.hq + head) * D;
  for (int t = wave; t < DT; t += NWV) {  // wave w finishes O^T tile w
    f32x16 acc[1] = {f32x16{}};
#pragma unroll
    for (int w = 0; w < NWV; ++w)
      acc[0] += wt[w] * *(const f32x16*)(smem + w * (DT * 4096 + 512) + t * 4096 + lane * 64);
    store_o_rows<1>(acc, inv, orow + 32 * t, hf, cvalid);
  }
  if (wave == 0 && hf == 0 && cvalid)
    p.lse[(int64_t)head * si.total_q + si.q0 + qrow] =
        L > 0.f ? (mmax * c + __log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// FP8 (OCP e4m3) inputs.  Same tiling and pipeline as the bf16 kernel, on the
// gfx950 fp8 MFMA v_mfma_scale_f32_32x32x64_f8f6f4 (block scales fixed at
// 2^0): each lane feeds 32 bytes of its row (A) or column (B); the 64 products
// pair A byte (half h, i) with B byte (half h, i), so any assignment of the 64
// keys (or head-dim entries) to (h, i) that both operands share is valid.
// Here byte i of half h is key / dim index 32h + i of the 64-wide chunk.
//  * S^T = K Q^T: K rows from LDS (two 16-byte reads), Q in registers.  The
//    K rows are placed in LDS so that accumulator register r of half h in
//    32-key sub-tile t holds key 32h + 16t + r: the exp'd scores are then
//    already the B operand of the P V product, bytes in key order.
//  * O^T += V^T P^T with P quantised to e4m3 (P <= 2^kLazy < 448); V^T
//    arrives through ds_read_b64_tr_b8, which hands lane i of each 16-lane
//    group column i of an 8-row x 16-byte block.
//  * O is normalised by the sum of the quantised weights that multiplied V,
//    taken on the matrix core as one more tile of the same product with an
//    all-ones A operand (every row of it is the column sum of P^T); the LSE
//    keeps the fp32 sum of the unquantised P.  With P taken against a stale
//    maximum even the largest weight of a row is rounded (3 mantissa bits),
//    and normalising by the unquantised sum would scale O by that rounding
//    (measured 7.9e-2 on rows spread over a few keys, against 3e-2 this way).
//  * The q and k descales fold into the exp2 scale (the forward-pass page's
//    FP8 branch multiplies softmax_scale_log2 by q_descale * k_descale); the
//    v descale multiplies O in the epilogue.
//  * XS (exact scores, opt-in): S^T = K Q^T on the bf16 MFMA instead, with
//    Q and K widened from e4m3 to bf16 (exactly: every e4m3 value is a bf16
//    value).  The fp8 matrix instruction keeps only about 13-14 bits below
//    the largest product of each dot product, so a row whose scores are far
//    above its other products loses precision in its LSE; the bf16 product is
//    exact.  K is widened per operand read (8 bytes -> 8 bf16, four
//    conversions), Q once per tile.  P V stays on the fp8 MFMA.

// LDS row of a K block (fp8) -> key: row 32t + rho holds key
// 32((rho>>2)&1) + 16t + 4(rho>>3) + (rho&3), i.e. the key of accumulator
// register r = 4(rho>>3) + (rho&3) of half (rho>>2)&1 in sub-tile t.
__device__ __forceinline__ int k8_lds_key(int row) {
  const int t = row >> 5, rho = row & 31;
  return 32 * ((rho >> 2) & 1) + 16 * t + 4 * (rho >> 3) + (rho & 3);
}
// 16-byte column swizzles of the fp8 K and V blocks (rows of D bytes):
//  * K: 16 consecutive rows read one column per LDS cycle;
//  * V: 8 consecutive rows x 32 contiguous bytes per half-wave transposed read.
template <int D>
__device__ __forceinline__ int swz_k8(int r) {
  return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int swz_v8(int r) {
  return D == 128 ? 2 * ((r >> 1) & 3) : 2 * ((r >> 2) & 1);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 (e4m3) for both operands, E8M0 block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four e4m3 ones (0x38 = 1.0) per dword: the A operand whose product with P^T
// is the column sum of P^T in every row.
constexpr int kE4m3OnesWord = 0x38383838;

// Eight e4m3 bytes -> eight bf16 values (exact).
__device__ __forceinline__ bf16x8 widen_e4m3(const u32x2 w) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int D, bool CAUSAL, bool XS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(Params p) {
  constexpr int TM = kTileM, TN = kTileN;
  constexpr int RB = D;                      // bytes per K/V row in LDS
  constexpr int BUF = TN * RB;               // bytes per K or V block buffer
  constexpr int CPR = D / 16;                // 16-byte chunks per row
  constexpr int NI = TN * CPR / 256;         // direct-load instructions per wave per block
  constexpr int KC = D / 64;                 // 64-wide k-chunks of the QK^T product
  constexpr int KC16 = D / 16;               // 16-wide k-chunks of the bf16 product (XS)
  constexpr int DT = D / 32;                 // 32-wide output tiles of O^T
  __shared__ __attribute__((aligned(1024))) char smem[4 * BUF];
  char* const kbuf0 = smem;
  char* const vbuf0 = smem + 2 * BUF;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  // ---- work item (as in the bf16 kernel)
  ItemIdx itx;
  if (!item_index(p, blockIdx.x, p.group, itx)) return;  // padding
  const int pair = itx.pair, mrev = itx.mrev;
  const int b = pair / p.hkv;
  const int head = (pair - b * p.hkv) * p.group + itx.hsub;
  const int mblk = CAUSAL ? (p.m_tiles - 1 - mrev) : mrev;
  const SeqInfo si = seq_info(p, b);
  const int m0 = mblk * TM;
  if (m0 >= si.sq) return;
  const int g = head / p.group;
  const int qi = m0 + wave * 32 + r32;
  const bool qvalid = qi < si.sq;

  const unsigned char* __restrict__ Q = (const unsigned char*)p.q;
  __bf16* __restrict__ O = (__bf16*)p.o;
  const float dq = p.descales[0], dk = p.descales[1], dvs = p.descales[2];
  const float c = p.scale_log2 * dq * dk;

  const int diag = si.sk - si.sq;
  int kend = si.sk;
  if (CAUSAL) kend = min(kend, m0 + TM + diag);
  const int nblk = kend > 0 ? (kend + TN - 1) / TN : 0;

  const int64_t qrow = ((int64_t)(si.q0 + qi) * p.hq + head) * D;  // elements of Q and O
  const int64_t lse_idx = (int64_t)head * si.total_q + si.q0 + qi;

  if (nblk == 0) {  // store_zero
    if (qvalid) {
      for (int e = hf * 4; e < D; e += 8) *(u32x2*)(O + qrow + e) = u32x2{0u, 0u};
      if (hf == 0) p.lse[lse_idx] = -INFINITY;
    }
    return;
  }

  // ---- Q fragments: lane holds Q[qi][64kc + 32hf .. +31]; XS: the e4m3
  // bytes Q[qi][16kc + 8hf .. +7] of the bf16 B operand of k-chunk kc,
  // widened where they are used (kept narrow: 16 registers instead of 32)
  i32x8 qf[XS ? 1 : KC];
  u32x2 qh[XS ? KC16 : 1];
  if constexpr (!XS) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const unsigned char* qp = Q + qrow + 64 * kc + 32 * hf;
      u32x4 lo = qvalid ? *(const u32x4*)qp : u32x4{0u, 0u, 0u, 0u};
      u32x4 hi = qvalid ? *(const u32x4*)(qp + 16) : u32x4{0u, 0u, 0u, 0u};
      qf[kc] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  } else {
#pragma unroll
    for (int kc = 0; kc < KC16; ++kc) {
      const unsigned char* qp = Q + qrow + 16 * kc + 8 * hf;
      qh[kc] = qvalid ? *(const u32x2*)qp : u32x2{0u, 0u};
    }
  }

  // ---- direct buffer -> LDS staging
  const int key_stride_b = p.hkv * D;  // bytes between consecutive keys
  const char* kseq = (const char*)p.k + ((int64_t)si.k0 * p.hkv + g) * D;
  const char* vseq = (const char*)p.v + ((int64_t)si.k0 * p.hkv + g) * D;
  unsigned koff[NI], voff[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int P = (wave * NI + u) * 64 + lane;
    const int row = P / CPR, pc = P % CPR;
    koff[u] = (unsigned)(k8_lds_key(row) * key_stride_b + ((pc ^ swz_k8<D>(row)) * 16));
    voff[u] = (unsigned)(row * key_stride_b + ((pc ^ swz_v8<D>(row)) * 16));
  }
  auto stage = [&](const char* seq, const unsigned* off, char* dst, int n) __attribute__((always_inline)) {
    const int keys_left = si.sk - n * TN;
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(seq + (int64_t)n * TN * key_stride_b), (short)0, keys_left * key_stride_b,
        kRsrcWord3);
#pragma unroll
    for (int u = 0; u < NI; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (wave * NI + u) * 1024), 16,
                                               off[u], 0, 0, 0);
  };
  auto stage_k = [&](int n, int buf) __attribute__((always_inline)) { stage(kseq, koff, kbuf0 + buf * BUF, n); };
  auto stage_v = [&](int n, int buf) __attribute__((always_inline)) { stage(vseq, voff, vbuf0 + buf * BUF, n); };

  // K operand: lane (r32, hf) of sub-tile t reads row 32t + r32, bytes
  // 64kc + 32hf .. +31 = logical 16-byte columns 4kc + 2hf and 4kc + 2hf + 1
  int ka[KC][2];
  {
    const int x = swz_k8<D>(r32);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int j = 0; j < 2; ++j) ka[kc][j] = r32 * RB + (((4 * kc + 2 * hf + j) ^ x) * 16);
  }
  // XS: the bf16 A operand of k-chunk kc is row 32t + r32, bytes 16kc + 8hf
  // .. +7, in logical 16-byte column kc
  auto k16_operand = [&](const char* kb, int t, int kc) __attribute__((always_inline)) {
    const int x = swz_k8<D>(r32);
    return widen_e4m3(*(const u32x2*)(kb + 32 * t * RB + r32 * RB + ((kc ^ x) * 16) + 8 * hf));
  };
  auto k_operand = [&](const char* kb, int t, int kc) __attribute__((always_inline)) {
    u32x4 lo = *(const u32x4*)(kb + 32 * t * RB + ka[kc][0]);
    u32x4 hi = *(const u32x4*)(kb + 32 * t * RB + ka[kc][1]);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // one of the score MFMAs: fp8 (step i of 2 * KC: k-chunk i >> 1, sub-tile
  // i & 1) or, XS, bf16 (step i of 2 * KC16)
  auto score_mfma = [&](const char* kb, f32x16* s, const int i) __attribute__((always_inline)) {
    const int kc = i >> 1, t = i & 1;
    if constexpr (!XS)
      s[t] = mfma_fp8(k_operand(kb, t, kc), qf[kc], s[t]);
    else
      s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k16_operand(kb, t, kc), widen_e4m3(qh[kc]),
                                                     s[t], 0, 0, 0);
  };
  constexpr int NSC = XS ? 2 * KC16 : 2 * KC;  // score MFMAs per block
  auto qk = [&](int buf, f32x16* s) __attribute__((always_inline)) {
    const char* kb = kbuf0 + buf * BUF;
#pragma unroll
    for (int t = 0; t < 2; ++t) s[t] = f32x16{};
#pragma unroll
    for (int i = 0; i < NSC; ++i) score_mfma(kb, s, i);
  };

  // V^T operand of dv tile dt: lane = 16G + 2t' + u reads 8 bytes of key row
  // 32(G>>1) + 8j + t' at dv columns 32dt + 16(G&1) + 8u (read j = 0..3); the
  // transpose hands lane i of the group column 32dt + 16(G&1) + i of those 8
  // rows: bytes 8j .. 8j+7 of its A operand (keys 32h + 8j + 0..7).
  int va[DT];
  {
    const int G = lane >> 4, s16 = lane & 15;
    const int tr = s16 >> 1, u = s16 & 1;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      va[t] = (32 * (G >> 1) + tr) * RB + ((((2 * t + (G & 1)) ^ swz_v8<D>(tr)) * 16)) + 8 * u;
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  // lq: the sum of the e4m3 weights that multiplied V (all 16 registers alike)
  f32x16 lq = f32x16{};
  i32x8 ones = {kE4m3OnesWord, kE4m3OnesWord, kE4m3OnesWord, kE4m3OnesWord,
                kE4m3OnesWord, kE4m3OnesWord, kE4m3OnesWord, kE4m3OnesWord};
  // opaque to the compiler, so that it keeps the operand in registers rather
  // than rebuilding it with seven moves for every block (measured 1.2-1.5 %)
  asm volatile("" : "+v"(ones));
  float m_run = -INFINITY;
  float l_run = 0.f;

  // Pipeline, buffer rotation and iteration pairs as in the bf16 kernel.
  f32x16 s_a[2], s_b[2];
  stage_k(nblk - 1, 0);
  stage_v(nblk - 1, 0);
  if (nblk >= 2) stage_k(nblk - 2, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  qk(0, s_a);

  auto iteration = [&](const int it, f32x16 (&sc)[2], f32x16 (&sn)[2],
                       const char* __restrict__ kread, const char* __restrict__ vread,
                       char* __restrict__ kdst, char* __restrict__ vdst,
                       auto mask_tag) __attribute__((always_inline)) {
    const int n = nblk - 1 - it;
    __syncthreads();
    if (n >= 2) stage(kseq, koff, kdst, n - 2);
    if (n >= 1) stage(vseq, voff, vdst, n - 1);

    // mask: key of register r of sub-tile t in half hf is n*TN + 32hf + 16t + r
    if (decltype(mask_tag)::value) {
      const int lim = CAUSAL ? min(si.sk - 1, qi + diag) : si.sk - 1;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (n * TN + 32 * hf + 16 * t + r > lim) sc[t][r] = -INFINITY;
    }

    // P = exp2(c*S - c*m) -> e4m3 bytes 16t + r of this half's B operand,
    // under the MFMAs of the next block's scores, against the running maximum
    // without the block's own: the pass stands when every lane's share of
    // the row sum is at most kLazyBound (so every P is within the bound the
    // lazy rescale keeps, below e4m3's largest value); otherwise -- a maximum
    // that grew, a row with no maximum yet -- the block maximum is taken, O
    // and l are rescaled to it where it grew, and P is computed again.
    float rs = 0.f;
    i32x8 pb;
    auto pword = [&](const float ms, const int w) __attribute__((always_inline)) {
      // dword w of P: bytes 4w .. 4w+3
      const int t = w >> 2, r0 = 4 * (w & 3);
      float pv[4], x0 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __builtin_fmaf(sc[t][r0 + e], c, -ms);
        if (e == 0) x0 = x;
        pv[e] = exp2_fast(x);
        // the sum starts from the block's first weight (0 + p is not folded)
        rs = (w == 0 && e == 0) ? pv[e] : rs + pv[e];
      }
      // The first conversion fills the word's low half and passes the high
      // half through from its third operand, which the second conversion
      // then overwrites: the dead exponent argument serves, where a constant
      // zero cost a register move per word (8 per block; measured +2.1 % on
      // causal fp8, +4 % non-causal)
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], __builtin_bit_cast(int, x0), false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], word, true);
      pb[w] = word;
    };
    if constexpr (!XS) {
#pragma unroll
      for (int t = 0; t < 2; ++t) sn[t] = f32x16{};
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        if ((w & 1) == 0 && (w >> 1) < NSC) score_mfma(kread, sn, w >> 1);
        pword(m_run * c, w);
      }
      // each of the four score MFMAs followed by a quarter of the softmax (8
      // exponentials, 16 other vector instructions); left to itself the
      // compiler groups the MFMAs after the softmax (measured 1.2 % slower)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sched_group(kSchedMfma, 1);
        sched_group(kSchedTrans, 8);
        sched_group(kSchedValu, 16);
      }
    } else {
      // the next block's scores after this block's P V (below): its tiles
      // then never live beside this block's, which keeps the kernel in 256
      // registers
#pragma unroll
      for (int w = 0; w < 8; ++w) pword(m_run * c, w);
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(rs <= kLazyBound)) != 0, 0)) {
      // The next block's scores are read on this (rare) path so that their
      // MFMAs stay where the schedule hints put them, among the exponentials:
      // otherwise the compiler sinks them past the branch, after the softmax
      // (non-causal +1.9 %; the causal kernel then runs out of registers)
      if constexpr (!CAUSAL && !XS) asm volatile("" ::"v"(sn[0]), "v"(sn[1]));
      const float m_new = fmax_nan(m_run, halfwave_max(block_max(sc)));
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
        const float alpha = m_new == -INFINITY ? 1.f : exp2_fast((m_run - m_new) * c);
        m_run = m_new;
        l_run *= alpha;
        lq *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
      }
      const float ms = (m_run == -INFINITY ? 0.f : m_run) * c;
      rs = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) pword(ms, w);
    }
    l_run += rs;

    // O^T += V_n^T P^T
    i32x8 va_op[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(vread + va[t]));
      i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(vread + 8 * RB + va[t]));
      i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(vread + 16 * RB + va[t]));
      i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(vread + 24 * RB + va[t]));
      va_op[t] = i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = mfma_fp8(va_op[t], pb, oacc[t]);
    lq = mfma_fp8(ones, pb, lq);
    if constexpr (XS) {
#pragma unroll
      for (int t = 0; t < 2; ++t) sn[t] = f32x16{};
#pragma unroll
      for (int i = 0; i < NSC; ++i) score_mfma(kread, sn, i);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  char* const k0b = kbuf0;
  char* const k1b = kbuf0 + BUF;
  char* const v0b = vbuf0;
  char* const v1b = vbuf0 + BUF;
  // masked iterations first, in a loop of their own (as in the bf16 kernel)
  const int thr = CAUSAL ? min(si.sk, m0 + diag + 1) : si.sk;
  const int n_plain = thr <= 0 ? 0 : min(nblk, thr / TN);  // blocks 0 .. n_plain-1 need no mask
  const int it_mask_end = min(nblk, (nblk - n_plain + 1) & ~1);
  int it = 0;
  for (; it < it_mask_end; it += 2) {
    iteration(it, s_a, s_b, k1b, v0b, k0b, v1b, BoolTag<true>{});
    if (it + 1 == nblk) {
      it = nblk;
      break;
    }
    iteration(it + 1, s_b, s_a, k0b, v1b, k1b, v0b, BoolTag<true>{});
  }
  for (; it < nblk; it += 2) {
    iteration(it, s_a, s_b, k1b, v0b, k0b, v1b, BoolTag<false>{});
    if (it + 1 == nblk) break;
    iteration(it + 1, s_b, s_a, k0b, v1b, k1b, v0b, BoolTag<false>{});
  }

  pin_accumulators(oacc);
  {
    f32x16 lqa[1] = {lq};
    pin_accumulators(lqa);
    lq = lqa[0];
  }
  const float l_tot = halfwave_sum(l_run);
  const float inv = l_tot > 0.f && lq[0] > 0.f ? dvs / lq[0] : 0.f;
  store_o_rows<DT>(oacc, inv, O + qrow, hf, qvalid);
  if (qvalid && hf == 0)
    p.lse[lse_idx] = l_tot > 0.f ? (m_run * c + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL>
void launch_fp8(const Launch& L, hipStream_t stream) {
  if (L.fp8_exact)
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, true>), dim3((unsigned)L.num_workgroups),
                       dim3(256), 0, stream, L.p);
  else
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, false>), dim3((unsigned)L.num_workgroups),
                       dim3(256), 0, stream, L.p);
}

template <int D, bool CAUSAL>
void launch_bf16_pp(const Launch& L, hipStream_t stream) {
  const dim3 grid((unsigned)L.num_workgroups), block(512);
  if (L.persist) {
    hipLaunchKernelGGL((fa_fwd_bf16_pp_persist_kernel<D, CAUSAL>), grid, block, 0, stream, L.p,
                       (int)L.num_items);
    return;
  }
  if (L.exp2_offload == 4)
    hipLaunchKernelGGL((fa_fwd_bf16_pp_kernel<D, CAUSAL, 4>), grid, block, 0, stream, L.p);
  else if (L.exp2_offload == 8)
    hipLaunchKernelGGL((fa_fwd_bf16_pp_kernel<D, CAUSAL, 8>), grid, block, 0, stream, L.p);
  else
    hipLaunchKernelGGL((fa_fwd_bf16_pp_kernel<D, CAUSAL, 0>), grid, block, 0, stream, L.p);
}

template <int D, bool CAUSAL>
void launch_bf16(const Launch& L, hipStream_t stream) {
  if (L.decode) {
    hipLaunchKernelGGL((fa_fwd_bf16_decode_kernel<D, CAUSAL>), dim3((unsigned)L.num_workgroups),
                       dim3(64 * kDecodeWaves), 0, stream, L.p);
    return;
  }
  if (L.pingpong) {
    launch_bf16_pp<D, CAUSAL>(L, stream);
    return;
  }
  if (L.query_tiles == 2)
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, 2>), dim3((unsigned)L.num_workgroups),
                       dim3(256), 0, stream, L.p);
  else
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, 1>), dim3((unsigned)L.num_workgroups),
                       dim3(256), 0, stream, L.p);
}

// AppendKV: copy the new K and V rows into the caches.  One thread moves 16
// bytes; thread i of the grid handles byte 16*(i % chunks) of new row
// i / chunks (rows ordered [b][j], K rows then V rows).
__global__ __launch_bounds__(256) void append_kv_kernel(Append a) {
  const int chunks = a.row_bytes / 16;
  const int64_t rows = (int64_t)a.batch * a.seqlen_new;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * rows * chunks) return;
  const int64_t r = i / chunks;
  const int ch = (int)(i - r * chunks);
  const bool is_v = r >= rows;
  const int64_t rr = is_v ? r - rows : r;
  const int b = (int)(rr / a.seqlen_new);
  const int j = (int)(rr - (int64_t)b * a.seqlen_new);
  const int pos = a.cache_seqlens[b] + j;
  if (pos < 0 || pos >= a.capacity) return;
  const char* src = (const char*)(is_v ? a.v_new : a.k_new) + rr * a.row_bytes + 16 * ch;
  char* dst = (char*)(is_v ? a.v_cache : a.k_cache) +
              ((int64_t)b * a.capacity + pos) * a.row_bytes + 16 * ch;
  *(u32x4*)dst = *(const u32x4*)src;
}

int device_is_gfx950() {
  // per device: 0 unknown, 1 yes, -1 no (atomic: host threads may launch
  // concurrently; a first query made twice stores the same answer)
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    const char* a = prop.gcnArchName;
    v = (a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' && a[5] == '0')
            ? 1 : -1;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1;
}

}  // namespace

int launch_append(const Append& A, void* stream_) {
  if (!device_is_gfx950()) return FA_ERR_DEVICE;
  const int64_t threads = 2 * (int64_t)A.batch * A.seqlen_new * (A.row_bytes / 16);
  if (threads == 0) return FA_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream_, A);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_DEVICE;
}

int launch(const Launch& L, void* stream_) {
  if (!device_is_gfx950()) return FA_ERR_DEVICE;
  hipStream_t stream = (hipStream_t)stream_;
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  if (L.fp8) {
    if (L.head_dim == 128) {
      if (L.causal) launch_fp8<128, true>(L, stream);
      else launch_fp8<128, false>(L, stream);
    } else {
      if (L.causal) launch_fp8<64, true>(L, stream);
      else launch_fp8<64, false>(L, stream);
    }
  } else if (L.head_dim == 128) {
    if (L.causal) launch_bf16<128, true>(L, stream);
    else launch_bf16<128, false>(L, stream);
  } else {
    if (L.causal) launch_bf16<64, true>(L, stream);
    else launch_bf16<64, false>(L, stream);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_DEVICE;
}

}  // namespace fa
