// fa_fwd_kernel.hip -- exact attention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup = 4 wavefronts = 128 query rows of one (sequence, head).
// Each wave owns 32 query rows and walks the key blocks (64 keys each) from
// the last admissible block down to the first, the block order of the
// consumer loop in "FlashAttention core algorithm: forward pass".
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
// K/V blocks are double-buffered in LDS and prefetched one block ahead into
// registers, so one barrier per block suffices.  The epilogue normalises by
// the row sum, writes O (bf16) and LSE (fp32, natural log), and writes
// O = 0 / LSE = -inf for rows with no admissible key -- the store_zero path
// of the page's epilogue.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_fwd.h"
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

// max / sum of a value over lanes l and l^32 (the two half-waves hold the
// same 32 queries): permlane32_swap returns {own, partner} in some order.
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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
  }
  return s;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_kernel(Params p) {
  constexpr int TM = kTileM, TN = kTileN;
  constexpr int KP = k_lds_pitch(D), VP = v_lds_pitch(D);
  constexpr int KBUF = TN * KP, VBUF = TN * VP;
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int NCH = TN * CPR / 256;        // chunks per thread per tile
  constexpr int KC = D / 16;                 // k-chunks of the QK^T product
  constexpr int DT = D / 32;                 // 32-wide output tiles of O^T
  __shared__ __attribute__((aligned(16))) char smem[kStages * (KBUF + VBUF)];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  // ---- work item: heaviest query tiles first (causal), then (batch, head)
  const int units = p.hq * p.batch;
  const int mrev = blockIdx.x / units;
  const int rest = blockIdx.x - mrev * units;
  const int head = rest % p.hq;
  const int b = rest / p.hq;
  const int mblk = CAUSAL ? (p.m_tiles - 1 - mrev) : mrev;
  const SeqInfo si = seq_info(p, b);
  const int m0 = mblk * TM;
  if (m0 >= si.sq) return;  // uniform over the workgroup, before any barrier
  const int g = head / p.group;
  const int qi = m0 + wave * 32 + r32;  // this lane's query row in the sequence
  const bool qvalid = qi < si.sq;

  const __bf16* __restrict__ Q = (const __bf16*)p.q;
  const __bf16* __restrict__ K = (const __bf16*)p.k;
  const __bf16* __restrict__ V = (const __bf16*)p.v;
  __bf16* __restrict__ O = (__bf16*)p.o;
  const float c = p.scale_log2;

  // ---- number of key blocks this tile needs
  const int diag = si.sk - si.sq;  // bottom-right alignment offset
  int kend = si.sk;
  if (CAUSAL) kend = min(kend, m0 + TM + diag);
  const int nblk = kend > 0 ? (kend + TN - 1) / TN : 0;

  const int64_t orow = ((int64_t)(si.q0 + qi) * p.hq + head) * D;
  const int64_t lse_idx = (int64_t)head * si.total_q + si.q0 + qi;

  if (nblk == 0) {  // no admissible key for any row of the tile
    if (qvalid) {
      for (int e = hf * 4; e < D; e += 8) *(u32x2*)(O + orow + e) = u32x2{0u, 0u};
      if (hf == 0) p.lse[lse_idx] = -INFINITY;
    }
    return;
  }

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds Q[qi][16kc + 8hf .. +7]
  bf16x8 qf[KC];
  {
    const __bf16* qp = Q + orow + 8 * hf;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 t = qvalid ? *(const u32x4*)(qp + 16 * kc) : u32x4{0u, 0u, 0u, 0u};
      qf[kc] = __builtin_bit_cast(bf16x8, t);
    }
  }

  // ---- K/V block staging: global -> registers -> LDS
  u32x4 kreg[NCH], vreg[NCH];
  auto load_tile = [&](int n) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int ch = tid + 256 * u;
      const int row = ch / CPR, col = ch % CPR;
      const int key = n * TN + row;
      const bool ok = key < si.sk;
      const int64_t off = ((int64_t)(si.k0 + key) * p.hkv + g) * D + col * 8;
      kreg[u] = ok ? *(const u32x4*)(K + off) : u32x4{0u, 0u, 0u, 0u};
      vreg[u] = ok ? *(const u32x4*)(V + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
    char* kb = smem + buf * (KBUF + VBUF);
    char* vb = kb + KBUF;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int ch = tid + 256 * u;
      const int row = ch / CPR, col = ch % CPR;
      *(u32x4*)(kb + k_lds_row(row) * KP + col * 16) = kreg[u];
      *(u32x4*)(vb + row * VP + col * 16) = vreg[u];
    }
  };

  // ---- running softmax state (per lane: one query, half of each key block)
  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // Transposed V reads: lane = 16G + i reads 8 bytes of key row
  // (kb + i/4) at dv columns 32dt + 16(G&1) + 4(i&3); after the transpose it
  // holds V[kb .. kb+3][32dt + 16(G&1) + i], i.e. its own A-operand column.
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;

  load_tile(nblk - 1);
  store_tile(0);
  if (nblk >= 2) load_tile(nblk - 2);

  for (int it = 0; it < nblk; ++it) {
    const int n = nblk - 1 - it;
    const int buf = it & 1;
    const char* kb = smem + buf * (KBUF + VBUF);
    const char* vb = kb + KBUF;
    __syncthreads();

    // S^T (two 32-key sub-tiles) = K_n Q^T
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x16{};
      const char* ka = kb + (32 * t + r32) * KP + hf * 16;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        bf16x8 a = *(const bf16x8*)(ka + kc * 32);
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], s[t], 0, 0, 0);
      }
    }

    // stage the next block while this one is consumed
    if (it + 1 < nblk) {
      store_tile(buf ^ 1);
      if (it + 2 < nblk) load_tile(n - 2);
    }

    // mask: key index of register r of sub-tile t is n*TN + 32t + 16(r/8) + 8hf + r%8
    const bool need_mask = (n + 1) * TN > si.sk || (CAUSAL && (n + 1) * TN - 1 > m0 + diag);
    if (need_mask) {
      const int lim = CAUSAL ? min(si.sk - 1, qi + diag) : si.sk - 1;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n * TN + 32 * t + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (key > lim) s[t][r] = -INFINITY;
        }
    }

    // online softmax, exp2 form
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = halfwave_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // all masked so far: keep P = 0
    const float ms = m_use * c;
    const float alpha = exp2_fast(m_run * c - ms);
    m_run = m_new;
    float rs = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_fast(__builtin_fmaf(s[t][r], c, -ms));
        rs += pv;
        pb[2 * t + (r >> 3)][r & 7] = (__bf16)pv;
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] *= alpha;

    // O^T += V_n^T P^T
#pragma unroll
    for (int kc2 = 0; kc2 < 4; ++kc2) {
      const char* vr = vb + (16 * kc2 + 8 * hf + tr_row) * VP + tr_col;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vr + t * 64));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vr + 4 * VP + t * 64));
        bf16x4 lob = __builtin_bit_cast(bf16x4, lo), hib = __builtin_bit_cast(bf16x4, hi);
        bf16x8 a = {lob[0], lob[1], lob[2], lob[3], hib[0], hib[1], hib[2], hib[3]};
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc2], oacc[t], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: normalise, O (bf16) and LSE (natural log)
  const float l_tot = halfwave_sum(l_run);
  if (!qvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 ov;
#pragma unroll
      for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(oacc[t][4 * i4 + j] * inv);
      *(bf16x4*)(O + orow + 32 * t + 8 * i4 + 4 * hf) = ov;
    }
  if (hf == 0) p.lse[lse_idx] = l_tot > 0.f ? (m_run * c + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL>
void launch_bf16(const Launch& L, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)L.num_workgroups), dim3(256), 0,
                     stream, L.p);
}

int device_is_gfx950() {
  static int cached[64];  // 0 unknown, 1 yes, -1 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    const char* a = prop.gcnArchName;
    cached[dev] = (a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' &&
                   a[5] == '0') ? 1 : -1;
  }
  return cached[dev] == 1;
}

}  // namespace

int launch(const Launch& L, void* stream_) {
  if (!device_is_gfx950()) return FA_ERR_DEVICE;
  hipStream_t stream = (hipStream_t)stream_;
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  if (L.fp8) return FA_ERR_UNSUPPORTED;
  if (L.head_dim == 128) {
    if (L.causal) launch_bf16<128, true>(L, stream);
    else launch_bf16<128, false>(L, stream);
  } else {
    if (L.causal) launch_bf16<64, true>(L, stream);
    else launch_bf16<64, false>(L, stream);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_DEVICE;
}

}  // namespace fa
