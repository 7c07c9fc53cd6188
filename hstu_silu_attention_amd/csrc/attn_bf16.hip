// Jagged target-aware causal SiLU attention on gfx950 (bf16 MFMA 32x32x16, float32
// accumulation). Scores never pass through a softmax: each history row sums
// SiLU(q.k) v over the keys at or before its position, each candidate over every
// history key plus itself, and the 1/max_len scale is applied once at the end.
#include "bf16_common.h"
#include "hstu_internal.h"

namespace hstu {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// One work item = (user, head, up to 128 query rows of one kind): four waves of QB
// blocks of 32 query rows each; two work items share a CU, so every SIMD runs two
// independent waves that hide each other's stalls. Keys advance 64 at a time through
// two LDS stages; K and V are staged row-major with 16-byte buffer loads whose range
// check returns zero for keys outside the user's [0, key_end).
//
// Per 32-key "half" h a wave computes, for each of its query blocks, S^T = K Q^T
// (queries along lanes), the bf16 weights a = SiLU(s), and O^T += V^T A^T; every K
// and V fragment read from LDS feeds all QB blocks. The V^T operand comes from the
// row-major V stage by the LDS transpose read: in each 16-lane group, lanes 4r..4r+3
// address 16 consecutive columns of key row r and lane i receives column i of those
// four rows. The key order inside the PV contraction is permuted to match the layout
// in which S^T's accumulators hold the weights; both operands use it.
//
// Software pipeline: step h issues the score MFMAs of half h + 1 and the PV MFMAs of
// half h - 1 while the VALU turns the scores of half h (finished in step h - 1) into
// weights, so no instruction of a step waits for another of the same step and the
// matrix and SiLU streams interleave. The loop body has no branches (a branch makes
// the register allocator copy the accumulators): every step of every wave does the
// same work, and masking is a wave-uniform bias inside the SiLU,
// SiLU(x) = x / (1 + 2^(x * -log2(e) + bias)), which is exactly x * sigmoid(x) for
// bias 0 and exactly 0 for bias +inf.
//
// History rows: keys are numbered from a shifted origin kappa = key + s with
// s = (-m) mod 32, so every wave's first query sits at a multiple of 32 and each
// query block meets the causal diagonal in exactly one half. Halves wholly before a
// block get bias 0; the diagonal half and every later one get +inf inside the loop,
// and a short pass after it adds the diagonal halves with a per-element mask.
// Candidate rows take bias 0 everywhere (keys past the last history key are zero, and
// SiLU(0) = 0) and add their own key in the epilogue.
//
// QB = 2 (64 rows per wave, one wave per SIMD, half the LDS reads per score) also
// compiles; on gfx950 it measured slower, a single wave per SIMD exposing its own
// dependency stalls.
//
// Row strides (measured with the LDS bank-conflict counter on gfx950): K rows of
// dh + 8 elements make the 16-byte fragment reads conflict-free; V rows need dh + 32
// for the transpose reads.
template <int DH>
struct AttnTile {
  static constexpr int WAVES = 4, NT = 64 * WAVES, QB = 1;
  static constexpr int BM = WAVES * QB * 32;     // query rows per work item
  static constexpr int KB = 64;                  // keys per LDS stage
  static constexpr int LDK = DH + 8, LDV = DH + 32;
  static constexpr int KSZ = KB * LDK, STAGE = KB * (LDK + LDV);
  static constexpr int CPR = DH / 8;             // 16-byte chunks per key row
  static constexpr int CPT = KB * CPR / NT;      // chunks per thread per matrix
  static constexpr int KK = DH / 16, MB = DH / 32;
};

constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw buffer, 32-bit data format

__device__ __forceinline__ float silu_bias(float x, float nlog2e, float bias) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(x, nlog2e, bias)));
}

template <int DH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_kernel(AttnArgs a) {
  using C = AttnTile<DH>;
  __shared__ __attribute__((aligned(16))) u16 smem[2 * C::STAGE];

  const int2 bin = a.bins[blockIdx.x % kXcds];
  if ((int)(blockIdx.x / kXcds) >= bin.y) return;
  const int4 t = a.tiles[bin.x + blockIdx.x / kXcds];
  const UserRec u = a.users[t.x];
  const int head = t.y >> 1, q0 = t.z, nq = t.w;
  const bool cand = (t.y & 1) != 0;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, so are the biases
  const int D = a.D;
  const size_t ld3 = 3 * (size_t)D;

  // this lane's two query rows (one per query block)
  bool qok[C::QB];
  size_t row[C::QB];
  bf16x8 qf[C::QB][C::KK];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int qloc = wv * 32 * C::QB + qb * 32 + l32;
    qok[qb] = qloc < nq;
    const int qi = q0 + (qok[qb] ? qloc : 0);
    row[qb] = cand ? (size_t)a.Nu + u.coff + qi : (size_t)u.uoff + qi;
    const u16* qrow = (const u16*)a.vqk + row[qb] * ld3 + D + head * DH;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
      qf[qb][kk] = as_bf16x8(qok[qb] ? *reinterpret_cast<const uint4*>(qrow + kk * 16 + hi * 8) : make_uint4(0, 0, 0, 0));
  }

  const int key_end = cand ? u.m + u.n : u.m + q0 + nq;  // keys [0, key_end)
  const int shift = cand ? 0 : (-u.m) & 31;               // kappa = key + shift
  const int nblk = (key_end + shift + C::KB - 1) / C::KB;
  const int wf = u.m + q0 + wv * 32 * C::QB + shift;              // kappa of this wave's first row (history)

  f32x16 oacc[C::QB][C::MB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[qb][mb][e] = 0.0f;

  // key row r of this user and head at byte offset 2 * (r * ld + col) of the resource;
  // rows outside [0, key_end) read as zero
  const int ld = (int)a.ld;
  const int nbytes = key_end * ld * 2;
  const __amdgpu_buffer_rsrc_t rk_src = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const u16*)a.kbase + (size_t)u.key_row * a.ld + head * DH), (short)0, nbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv_src = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const u16*)a.vbase + (size_t)u.key_row * a.ld + head * DH), (short)0, nbytes, kBufferWord3);
  auto load_row_chunk = [&](const __amdgpu_buffer_rsrc_t& src, int key, int col) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(src, (key * ld + col) * 2, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };

  // staging: thread t moves chunk t + NT*i (i < CPT): key row c / CPR, column (c % CPR) * 8
  uint4 rk[C::CPT], rv[C::CPT];
  auto fetch = [&](int blk) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + C::NT * i, key = blk * C::KB + c / C::CPR - shift, col = (c % C::CPR) * 8;
      rk[i] = load_row_chunk(rk_src, key, col);
      rv[i] = load_row_chunk(rv_src, key, col);
    }
  };
  auto store = [&](int stage) {
    u16* sk = smem + stage * C::STAGE;
    u16* sv = sk + C::KSZ;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + C::NT * i, r = c / C::CPR, col = (c % C::CPR) * 8;
      *reinterpret_cast<uint4*>(sk + r * C::LDK + col) = rk[i];
      *reinterpret_cast<uint4*>(sv + r * C::LDV + col) = rv[i];
    }
  };

  // LDS fragments: K rows for the scores, V^T columns for PV (weight chunk c, element
  // e <-> key 16c + 8*(e/4) + 4*hi + e%4 of the half; the transpose reads fetch V rows
  // 16c + 4*hi + r and + 8)
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto read_k_at = [&](const u16* rows, bf16x8 (&kf)[C::KK]) {   // rows: key row 0 of the half
    const u16* sk = rows + l32 * C::LDK + hi * 8;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) kf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(sk + kk * 16));
  };
  auto read_v_at = [&](const u16* rows, bf16x8 (&vf)[2][C::MB]) {
    const u16* sv = rows + tr_row * C::LDV + tr_col;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const u16* p = sv + 16 * c * C::LDV + mb * 32;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 8 * C::LDV));
        vf[c][mb] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  // half h lives in stage (h / 2) % 2 at rows 32 * (h % 2) ("half -1": stage 1, rows 32..)
  auto k_rows = [&](int h) { return smem + ((h >> 1) & 1) * C::STAGE + (h & 1) * 32 * C::LDK; };
  auto v_rows = [&](int h) { return smem + ((h >> 1) & 1) * C::STAGE + C::KSZ + (h & 1) * 32 * C::LDV; };

  // S^T = K Q^T for query block qb; s[4*i + j] = q . k(key 8*i + 4*hi + j of the half)
  auto score_mfma = [&](const bf16x8 (&kf)[C::KK], int qb, f32x16& s) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) s = mfma32(kf[kk], qf[qb][kk], s);
  };
  auto pv_mfma = [&](const bf16x8 (&vf)[2][C::MB], int qb, const bf16x8 (&w)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) oacc[qb][mb] = mfma32(vf[c][mb], w[c], oacc[qb][mb]);
  };

  const float nlog2e = -1.4426950408889634f;
  const float kInf = __builtin_huge_valf();
  // bias of query block qb in half h: 0 for halves wholly before the block's first row
  auto bias = [&](int h, int qb) { return cand || wf + 32 * qb - 32 * h > 0 ? 0.0f : kInf; };

  // Step h: (si, wi) = scores of half h, weights of half h - 1 -> (so, wo) = scores of
  // half h + 1, weights of half h.
  auto body = [&](int h, const f32x16 (&si)[C::QB], const bf16x8 (&wi)[C::QB][2], f32x16 (&so)[C::QB], bf16x8 (&wo)[C::QB][2]) {
    bf16x8 kf[C::KK], vf[2][C::MB];
    read_k_at(k_rows(h + 1), kf);
    read_v_at(v_rows(h - 1), vf);
    __builtin_amdgcn_sched_barrier(0);   // every fragment read goes out before the step's math
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) score_mfma(kf, qb, so[qb]);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) pv_mfma(vf, qb, wi[qb]);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const float b = bias(h, qb);
#pragma unroll
      for (int e = 0; e < 16; ++e) wo[qb][e >> 3][e & 7] = (__bf16)silu_bias(si[qb][e], nlog2e, b);
    }
    // SiLU work first (its inputs are ready while the reads are in flight), then each
    // MFMA followed by a share of the rest
    constexpr unsigned MFMA = 0x008, VALU = 0x002;
    constexpr int kMfma = C::QB * (C::KK + 2 * C::MB);
    __builtin_amdgcn_sched_group_barrier(VALU, 16, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(VALU, 5, 0);
    }
  };

  // V rows of "half -1" are multiplied by the zero weights of the first step: make
  // them finite
  {
    u16* sv = smem + C::STAGE + C::KSZ;
    for (int i = tid; i < C::KB * C::LDV / 8; i += C::NT) *reinterpret_cast<uint4*>(sv + 8 * i) = make_uint4(0, 0, 0, 0);
  }
  fetch(0);
  store(0);
  __syncthreads();
  // ping-pong state: (sA, wA) enters the even steps, (sB, wB) the odd ones
  f32x16 sA[C::QB], sB[C::QB];
  bf16x8 wA[C::QB][2], wB[C::QB][2];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) wA[qb][0] = wA[qb][1] = as_bf16x8(make_uint4(0, 0, 0, 0));
  {
    bf16x8 kf[C::KK];
    read_k_at(k_rows(0), kf);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) score_mfma(kf, qb, sA[qb]);
  }
  for (int b = 0; b < nblk; ++b) {
    // the last block re-fetches itself into the idle stage (unconditional steps keep
    // the loop body free of branches)
    fetch(b + 1 < nblk ? b + 1 : b);
    body(2 * b, sA, wA, sB, wB);       // K of block b, V of block b - 1
    __syncthreads();                   // every wave is past its reads of block b - 1
    store((b + 1) & 1);
    __syncthreads();                   // block b + 1 visible
    body(2 * b + 1, sB, wB, sA, wA);   // K of block b + 1, V of block b
  }
  if (nblk > 0) {
    // PV of the last half (its weights are in wA)
    bf16x8 vf[2][C::MB];
    read_v_at(v_rows(2 * nblk - 1), vf);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) pv_mfma(vf, qb, wA[qb]);
  }

  if (!cand) {
    // The diagonal half of each history block, in a private LDS area per wave: key
    // offset j of the half is visible to row offset i when j <= i.
    u16* dk = smem + wv * 32 * (C::LDK + C::LDV);
    u16* dv = dk + 32 * C::LDK;
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      __syncthreads();   // the stages (or the previous block's area) are free
      const int k0 = wf + 32 * qb - shift;   // key of the half's first row
#pragma unroll
      for (int i = 0; i < C::CPR / 2; ++i) {
        const int c = lane + 64 * i, r = c / C::CPR, col = (c % C::CPR) * 8;
        *reinterpret_cast<uint4*>(dk + r * C::LDK + col) = load_row_chunk(rk_src, k0 + r, col);
        *reinterpret_cast<uint4*>(dv + r * C::LDV + col) = load_row_chunk(rv_src, k0 + r, col);
      }
      __syncthreads();
      bf16x8 kf[C::KK], vf[2][C::MB], w[2];
      f32x16 s;
      read_k_at(dk, kf);
      score_mfma(kf, qb, s);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = 8 * (e >> 2) + 4 * hi + (e & 3);
        w[e >> 3][e & 7] = (__bf16)silu_bias(s[e], nlog2e, j <= l32 ? 0.0f : kInf);
      }
      read_v_at(dv, vf);
      pv_mfma(vf, qb, w);
    }
  }

#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const u16* vqk = (const u16*)a.vqk + row[qb] * ld3 + head * DH;   // V | Q | K of this row
    if (cand) {
      // the candidate's own key and value: a_self = bf16(SiLU(q . k_self))
      float part = 0.0f;
      if (qok[qb]) {
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
          const uint4 kv = *reinterpret_cast<const uint4*>(vqk + 2 * D + kk * 16 + hi * 8);
          const uint32_t wds[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            part += (float)qf[qb][kk][2 * e] * bf2f_lo(wds[e]);
            part += (float)qf[qb][kk][2 * e + 1] * bf2f_hi(wds[e]);
          }
        }
      }
      const float dot = part + __shfl_xor(part, 32);
      const float as = qok[qb] ? round_bf(silu(dot)) : 0.0f;
      if (qok[qb]) {
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint2 vv = *reinterpret_cast<const uint2*>(vqk + mb * 32 + i * 8 + hi * 4);
            oacc[qb][mb][4 * i + 0] += as * bf2f_lo(vv.x);
            oacc[qb][mb][4 * i + 1] += as * bf2f_hi(vv.x);
            oacc[qb][mb][4 * i + 2] += as * bf2f_lo(vv.y);
            oacc[qb][mb][4 * i + 3] += as * bf2f_hi(vv.y);
          }
      }
    }
    if (qok[qb]) {
      // O = bf16(inv * acc) into columns [D, 2D) of the output GEMM's operand row
      u16* orow = (u16*)a.aout + row[qb] * ld3 + D + head * DH;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float o0 = a.inv * oacc[qb][mb][4 * i + 0], o1 = a.inv * oacc[qb][mb][4 * i + 1];
          const float o2 = a.inv * oacc[qb][mb][4 * i + 2], o3 = a.inv * oacc[qb][mb][4 * i + 3];
          *reinterpret_cast<uint2*>(orow + mb * 32 + i * 8 + hi * 4) = make_uint2(pack2(o0, o1), pack2(o2, o3));
        }
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(int dh, const AttnArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (dh == 64)
    attn_kernel<64><<<grid, AttnTile<64>::NT, 0, s>>>(a);
  else if (dh == 128)
    attn_kernel<128><<<grid, AttnTile<128>::NT, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int attn_block_rows_bf16() { return AttnTile<128>::BM; }

}  // namespace hstu
