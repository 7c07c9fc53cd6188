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

// One work item = (user, head, up to 128 query rows of one kind): four waves of 32
// query rows. Keys advance 64 at a time through two LDS stages; K and V are both
// staged row-major with 16-byte loads (keys past the user's last one are zero).
//
// Per 32-key half a wave computes S^T = K Q^T (queries along lanes), turns it into
// bf16 weights a = SiLU(s) (masked only in blocks that cross the causal diagonal or
// the last key), then O^T += V^T A^T. The V^T operand comes from the row-major V
// stage by the LDS transpose read: in each 16-lane group, lanes 4r..4r+3 address
// 16 consecutive columns of key row r and lane i receives column i of those four
// rows. The key order inside the PV contraction is permuted to match the layout in
// which S^T's accumulators hold the weights; both operands use the same order.
//
// Row strides (measured with the LDS bank-conflict counter on gfx950): K rows of
// dh + 8 elements make the 16-byte fragment reads conflict-free; V rows need dh + 32
// for the transpose reads (dh + 16 costs about two cycles per read).
template <int DH>
struct AttnTile {
  static constexpr int BM = 128, KB = 64;
  static constexpr int LDK = DH + 8, LDV = DH + 32;
  static constexpr int KSZ = KB * LDK, STAGE = KB * (LDK + LDV);
  static constexpr int CPR = DH / 8;             // 16-byte chunks per key row
  static constexpr int CPT = KB * CPR / 256;     // chunks per thread per matrix
};

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
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int D = a.D;
  const size_t ld3 = 3 * (size_t)D;
  const int qloc = wv * 32 + l32;
  const bool qok = qloc < nq;
  const int qi = q0 + (qok ? qloc : 0);
  const size_t row = cand ? (size_t)a.Nu + u.coff + qi : (size_t)u.uoff + qi;
  const u16* vqk = (const u16*)a.vqk + row * ld3 + head * DH;   // V | Q | K of this row and head

  bf16x8 qf[DH / 16];
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk)
    qf[kk] = as_bf16x8(qok ? *reinterpret_cast<const uint4*>(vqk + D + kk * 16 + hi * 8) : make_uint4(0, 0, 0, 0));

  const int key_end = cand ? u.m + u.n : u.m + q0 + nq;  // keys [0, key_end)
  const int qpos = u.m + qi;                             // history row: keys <= qpos
  // This wave's query positions (history items): the block loop skips key blocks
  // past its last query and drops the mask for blocks before its first one.
  const bool wave_live = wv * 32 < nq;
  const int wq_first = u.m + q0 + wv * 32;
  const int wq_last = u.m + q0 + min(nq, wv * 32 + 32) - 1;

  f32x16 oacc[DH / 32];
#pragma unroll
  for (int mb = 0; mb < DH / 32; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[mb][e] = 0.0f;

  // staging: thread t moves chunk t + 256*i (i < CPT): key row c / CPR, column (c % CPR) * 8
  const u16* kp = (const u16*)a.kbase + (size_t)u.key_row * a.ld + head * DH;
  const u16* vp = (const u16*)a.vbase + (size_t)u.key_row * a.ld + head * DH;
  uint4 rk[C::CPT], rv[C::CPT];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + 256 * i, key = k0 + c / C::CPR, col = (c % C::CPR) * 8;
      const bool in = key < key_end;
      rk[i] = in ? *reinterpret_cast<const uint4*>(kp + (size_t)key * a.ld + col) : make_uint4(0, 0, 0, 0);
      rv[i] = in ? *reinterpret_cast<const uint4*>(vp + (size_t)key * a.ld + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int stage) {
    u16* sk = smem + stage * C::STAGE;
    u16* sv = sk + C::KSZ;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + 256 * i, r = c / C::CPR, col = (c % C::CPR) * 8;
      *reinterpret_cast<uint4*>(sk + r * C::LDK + col) = rk[i];
      *reinterpret_cast<uint4*>(sv + r * C::LDV + col) = rv[i];
    }
  };

  // transpose-read lane constants: group g = lane / 16 reads key rows 4*(g/2) + r
  // (r = (lane % 16) / 4) at columns 16*(g%2) + 4*(lane % 4)
  const int tr_row = 4 * hi + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  const int nblk = (key_end + C::KB - 1) / C::KB;
  if (nblk > 0) {
    fetch(0);
    store(0);
  }
  __syncthreads();
  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * C::KB;
    // the last block re-fetches itself into the idle stage (unconditional steps keep
    // the prefetch registers free of loop-carried state)
    fetch(kb + 1 < nblk ? k0 + C::KB : k0);
    const u16* sk = smem + (kb & 1) * C::STAGE;
    const u16* sv = sk + C::KSZ;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int kbase = k0 + kh * 32;
      const bool live = cand ? kbase < key_end : (wave_live && kbase <= wq_last);
      if (live) {
        const bool full = cand ? (kbase + 32 <= key_end) : (kbase + 31 <= wq_first);
        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk) {
          const bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4*>(sk + (kh * 32 + l32) * C::LDK + kk * 16 + hi * 8));
          s = mfma32(kf, qf[kk], s);
        }
        // s[4*i + j] = q(row l32) . k(key kbase + 8*i + 4*hi + j)
        bf16x8 af[2];
        if (full) {
#pragma unroll
          for (int e = 0; e < 16; ++e) af[e >> 3][e & 7] = (__bf16)silu(s[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kbase + (e >> 2) * 8 + hi * 4 + (e & 3);
            const bool ok = cand ? key < key_end : key <= qpos;
            af[e >> 3][e & 7] = (__bf16)(ok ? silu(s[e]) : 0.0f);
          }
        }
        // weight chunk c, element e <-> key kbase + 16c + 8*(e/4) + 4*hi + e%4: the
        // transpose reads fetch V rows kbase + 16c + 4*hi + r and the same + 8
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u16* vrow = sv + (kh * 32 + 16 * c + tr_row) * C::LDV + tr_col;
#pragma unroll
          for (int mb = 0; mb < DH / 32; ++mb) {
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vrow + mb * 32));
            const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vrow + 8 * C::LDV + mb * 32));
            const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[mb] = mfma32(vf, af[c], oacc[mb]);
          }
        }
      }
    }
    store((kb + 1) & 1);
    __syncthreads();
  }

  if (cand) {
    // the candidate's own key and value: a_self = bf16(SiLU(q . k_self))
    const u16* krow = vqk + 2 * D;
    const u16* vrow = vqk;
    float part = 0.0f;
    if (qok) {
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + kk * 16 + hi * 8);
        const uint32_t wds[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part += (float)qf[kk][2 * e] * bf2f_lo(wds[e]);
          part += (float)qf[kk][2 * e + 1] * bf2f_hi(wds[e]);
        }
      }
    }
    const float dot = part + __shfl_xor(part, 32);
    const float as = qok ? round_bf(silu(dot)) : 0.0f;
    if (qok) {
#pragma unroll
      for (int mb = 0; mb < DH / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint2 vv = *reinterpret_cast<const uint2*>(vrow + mb * 32 + i * 8 + hi * 4);
          oacc[mb][4 * i + 0] += as * bf2f_lo(vv.x);
          oacc[mb][4 * i + 1] += as * bf2f_hi(vv.x);
          oacc[mb][4 * i + 2] += as * bf2f_lo(vv.y);
          oacc[mb][4 * i + 3] += as * bf2f_hi(vv.y);
        }
    }
  }
  if (qok) {
    // O = bf16(inv * acc) into columns [D, 2D) of the output GEMM's operand row, and the
    // gate bf16(U * O), from this row's U (columns [0, D)), into columns [2D, 3D)
    u16* arow = (u16*)a.aout + row * ld3 + head * DH;
    uint2 uv[DH / 32][4];
#pragma unroll
    for (int mb = 0; mb < DH / 32; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) uv[mb][i] = *reinterpret_cast<const uint2*>(arow + mb * 32 + i * 8 + hi * 4);
#pragma unroll
    for (int mb = 0; mb < DH / 32; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o0 = round_bf(a.inv * oacc[mb][4 * i + 0]), o1 = round_bf(a.inv * oacc[mb][4 * i + 1]);
        const float o2 = round_bf(a.inv * oacc[mb][4 * i + 2]), o3 = round_bf(a.inv * oacc[mb][4 * i + 3]);
        const int c = mb * 32 + i * 8 + hi * 4;
        *reinterpret_cast<uint2*>(arow + D + c) = make_uint2(pack2(o0, o1), pack2(o2, o3));
        const uint2 g = make_uint2(pack2(bf2f_lo(uv[mb][i].x) * o0, bf2f_hi(uv[mb][i].x) * o1),
                                   pack2(bf2f_lo(uv[mb][i].y) * o2, bf2f_hi(uv[mb][i].y) * o3));
        *reinterpret_cast<uint2*>(arow + 2 * D + c) = g;
      }
  }
}

}  // namespace

hipError_t launch_attn_bf16(int dh, const AttnArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (dh == 64)
    attn_kernel<64><<<grid, 256, 0, s>>>(a);
  else if (dh == 128)
    attn_kernel<128><<<grid, 256, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int attn_block_rows_bf16() { return AttnTile<128>::BM; }

}  // namespace hstu
