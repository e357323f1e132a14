// Prefill: causal cross-attention of every prompt row, bf16 storage, MFMA.
//
// Attn_l = softmax(Q^l K^T * scale + M_causal) V^ over the whole prompt (page
// "YOCO", section "Cross-Decoder", Attn_l equation; causal rule j <= i from
// section "架构总览"). A dense contraction: both products run on
// v_mfma_f32_32x32x16_bf16.
//
// Workgroup = W waves x 32 query rows. The rows of one workgroup belong to one
// KV head: up to W query heads of its group at the same 32 positions (or fewer
// heads over more positions), so every K^/V^ tile staged in LDS serves all of
// them. Per 64-key tile and per wave:
//   S^T[key][query] = K^ . Q^T      A = K^ rows from LDS, B = Q^T in registers
//   online softmax on S^T           one query per lane pair (lane, lane ^ 32)
//   O^T[dim][query] += V^T . P^T    B = P^T straight from the S^T registers,
//                                   A = V^T from an LDS tile stored transposed
// The accumulator layout of a 32x32 MFMA gives lane l the keys
// 8*(r/4) + 4*(l/32) + (r%4) of query l%32; taking registers 8c..8c+7 as the
// B operand of the PV step c means the step's k-slot e of lane half h is key
// 16c + 8*(e/4) + 4h + (e%4). The V^T tile stores key k at column k with bits
// 2 and 3 swapped, which makes those eight keys one contiguous 16-byte read.
// LDS rows are padded by 16 bytes, so that the 16-byte reads of 8 (or 16)
// consecutive lanes from 8 (16) consecutive rows hit distinct banks.
// Tiles wholly above the diagonal are never loaded; diagonal tiles are masked.
// Grid: one workgroup per (unit, position block), a unit being a (sequence, KV
// head, head chunk); position blocks run longest first. Workgroups reach the 8
// XCDs round-robin by index, and prefill_schedule (internal.h) orders them so
// that each XCD walks whole units (or a share of one unit's blocks when there
// are fewer than 8 units): the workgroups resident on one XCD then stream the
// same K^/V^ rows through that XCD's L2.
#include <hip/hip_bf16.h>

#include "internal.h"

namespace yoco {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBN = 64;          // keys per tile
constexpr int kKPad = 8;         // bf16 padding per K^ row in LDS
constexpr int kVPad = 8;         // bf16 padding per V^T row in LDS

__device__ __forceinline__ int swap_bits_2_3(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

template <int D>
struct TileRegs {
  static constexpr int kChunks = (kBN * D / 8 + kPrefillThreads - 1) / kPrefillThreads;  // 16-byte K^ chunks per thread
  static constexpr int kVBlocks = ((kBN / 4) * (D / 8) + kPrefillThreads - 1) / kPrefillThreads;  // 4-key x 8-dim V^ blocks
  u32x4 k[kChunks];       // native vectors: HIP's uint4 struct is copied by memcpy, which
  u32x4 v[kVBlocks][4];   // keeps an array of it out of registers
};

// Loads are unconditional (indices wrap onto valid chunks when a tile has fewer
// chunks than threads, and only the LDS store is guarded): a conditionally
// assigned register tile would be demoted to scratch memory.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const __bf16* kbase, const __bf16* vbase,
                                          int64_t row_stride, int key0, int last) {
  constexpr int kKChunks = kBN * D / 8;
  constexpr int kVBlocksAll = (kBN / 4) * (D / 8);
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kChunks; ++i) {
    const int c = (t + kPrefillThreads * i) % kKChunks;
    int key = key0 + c / (D / 8);
    key = key < last ? key : last;
    r.k[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * row_stride + 8 * (c % (D / 8)));
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kVBlocks; ++i) {
    const int c = (t + kPrefillThreads * i) % kVBlocksAll;
    const int kg = c % (kBN / 4);   // key group fastest: see store_tile
    const int dc = c / (kBN / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int key = key0 + 4 * kg + j;
      key = key < last ? key : last;
      r.v[i][j] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * row_stride + 8 * dc);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, __bf16* ks, __bf16* vts) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kChunks; ++i) {
    const int c = t + kPrefillThreads * i;
    if (c < kBN * D / 8)
      *reinterpret_cast<u32x4*>(ks + (c / (D / 8)) * (D + kKPad) + 8 * (c % (D / 8))) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kVBlocks; ++i) {
    const int c = t + kPrefillThreads * i;
    if (c < (kBN / 4) * (D / 8)) {
      // 16 consecutive lanes hold the 16 key groups of one 8-dim block: each
      // 8-byte store of theirs fills one 128-byte V^T row without bank conflicts
      const int kg = c % (kBN / 4);
      const int dc = c / (kBN / 4);
      const int kcol = swap_bits_2_3(4 * kg);   // 4 consecutive keys stay consecutive
      // element access on register vectors (a pointer cast would force the tile to scratch)
      const u32x4 a0 = r.v[i][0], a1 = r.v[i][1], a2 = r.v[i][2], a3 = r.v[i][3];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint2 even, odd;
        even.x = (a0[w] & 0xffffu) | (a1[w] << 16);
        even.y = (a2[w] & 0xffffu) | (a3[w] << 16);
        odd.x = (a0[w] >> 16) | (a1[w] & 0xffff0000u);
        odd.y = (a2[w] >> 16) | (a3[w] & 0xffff0000u);
        const int d = 8 * dc + 2 * w;
        *reinterpret_cast<uint2*>(vts + d * (kBN + kVPad) + kcol) = even;
        *reinterpret_cast<uint2*>(vts + (d + 1) * (kBN + kVPad) + kcol) = odd;
      }
    }
  }
}

// Running-max slack (base 2): the O accumulator is rescaled only when a tile's
// max exceeds the reference by more than this, so P <= 2^8 between rescales.
constexpr float kRescaleSlack = 8.0f;

// One 64-key tile for one wave: S^T = K^ Q^T, online softmax, O^T += V^T P^T.
template <int D, bool MASK>
__device__ __forceinline__ void tile_step(const __bf16* ks, const __bf16* vts, const bf16x8 (&qf)[D / 16],
                                          f32x16 (&acc)[D / 32], float& m, float& l, int key0, int my_pos,
                                          int n_kv, float c, int qj, int hf) {
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    const __bf16* krow = ks + (kb * 32 + qj) * (D + kKPad) + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * kk);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (MASK) {
        const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key > my_pos || key >= n_kv) s[kb][r] = -INFINITY;
      }
      mx = fmaxf(mx, s[kb][r]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mx2 = mx * c;  // c > 0: the max commutes with the scale
  const bool grow = mx2 > m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    // only the lanes whose own max grew move their reference: every row's
    // arithmetic stays independent of the other rows in the wave
    const float m_new = grow ? mx2 : m;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;  // exp2(-inf) = 0 on the first tile
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
  }
  const float neg_m = m == -INFINITY ? 0.f : -m;
  bf16x8 pf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * cc + 2 * i], c, neg_m));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * cc + 2 * i + 1], c, neg_m));
        w[i] = pack2(e0, e1);
        l += e0 + e1;   // fp32 sum of the unrounded weights keeps the LSE fp32-accurate
      }
      pf[kb][cc] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const __bf16* vrow = vts + (32 * t + qj) * (kBN + kVPad) + 8 * hf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + 32 * kb + 16 * cc);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][cc], acc[t], 0, 0, 0);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_bf16_kernel(AttnParams p) {
  // two K^ tiles then two V^T tiles; the output staging of the epilogue reuses the start
  constexpr int kKTile = kBN * (D + kKPad);
  constexpr int kVTile = D * (kBN + kVPad);
  constexpr int kOStride = D + 8;
  static_assert(kPrefillWaves * kPrefillRowsPerWave * kOStride <= 2 * (kKTile + kVTile), "staging fits");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (kKTile + kVTile)];
  auto ks_lds = [&](int b) { return smem + b * kKTile; };
  auto vt_lds = [&](int b) { return smem + 2 * kKTile + b * kVTile; };

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int qj = lane & 31;   // query column of this lane in S^T / O^T tiles
  const int hf = lane >> 5;   // lane half

  const int hpw = prefill_heads_per_wg(p.group);
  const int ppw = kPrefillWaves / hpw;
  const int hchunks = p.group / hpw;
  const int units = p.batch * p.hkv * hchunks;
  int unit, rank;
  prefill_schedule(blockIdx.x, units, p.pos_blocks, &unit, &rank);
  const int hc = unit % hchunks;
  const int kh = (unit / hchunks) % p.hkv;
  const int b = unit / (hchunks * p.hkv);
  const int h = kh * p.group + hc * hpw + wave % hpw;   // this wave's query head
  const int pbl = wave / hpw;                          // this wave's position block inside the WG
  const int pos_per_wg = kPrefillRowsPerWave * ppw;
  const float c = p.scale_log2;
  if (rank >= p.pos_blocks) return;

  int64_t start;
  const int32_t n_kv = readable_rows(p.seq_start, p.seq_len, p.seq_cap, p.pool_rows, b, &start);
  int64_t q0 = p.cu_seqlens[b];
  int64_t q1 = p.cu_seqlens[b + 1];
  if (q1 > p.total_q) q1 = p.total_q;
  if (q0 < 0 || q0 > q1) return;
  const int32_t n_q = (int32_t)(q1 - q0);
  const int32_t offset = n_kv > n_q ? n_kv - n_q : 0;

  const int64_t row_stride = (int64_t)p.hkv * D;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + start * row_stride + (int64_t)kh * D;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + start * row_stride + (int64_t)kh * D;
  const __bf16* qbase = static_cast<const __bf16*>(p.q);

  for (int pw = p.pos_blocks - 1 - rank; pw >= 0 && pw * pos_per_wg < n_q; pw += p.pos_blocks) {
    const int r0 = pw * pos_per_wg + pbl * kPrefillRowsPerWave;   // first row of this wave
    const int wg_last_row = min(n_q, (pw + 1) * pos_per_wg) - 1;
    const int wg_last_key = min(wg_last_row + offset, n_kv - 1);
    const int n_tiles = wg_last_key >= 0 ? wg_last_key / kBN + 1 : 0;
    const bool wave_active = r0 < n_q;
    const int wave_min_pos = r0 + offset;
    const int wave_max_pos = min(r0 + kPrefillRowsPerWave, n_q) - 1 + offset;
    // tiles [0, full_tiles) are visible to every row of the wave: no mask
    const int full_tiles = min((wave_min_pos + 1) / kBN, n_kv / kBN);
    const int my_row = min(r0 + qj, n_q - 1);
    const int my_pos = r0 + qj + offset;

    // Q^T as the B operand: query my_row, dims 16*kk + 8*hf .. +8
    bf16x8 qf[D / 16];
    {
      const __bf16* qsrc = qbase + ((q0 + my_row) * p.hq + h) * D + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qsrc + 16 * kk));
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    float m = -INFINITY, l = 0.f;

    TileRegs<D> regs;
    if (n_tiles > 0) {
      load_tile<D>(regs, kbase, vbase, row_stride, 0, n_kv - 1);
      store_tile<D>(regs, ks_lds(0), vt_lds(0));
    }
    __syncthreads();
    for (int kt = 0; kt < n_tiles; ++kt) {
      const int buf = kt & 1;
      const bool more = kt + 1 < n_tiles;
      if (more) load_tile<D>(regs, kbase, vbase, row_stride, (kt + 1) * kBN, n_kv - 1);
      const int key0 = kt * kBN;
      if (wave_active && key0 <= wave_max_pos) {
        if (kt < full_tiles)
          tile_step<D, false>(ks_lds(buf), vt_lds(buf), qf, acc, m, l, key0, my_pos, n_kv, c, qj, hf);
        else
          tile_step<D, true>(ks_lds(buf), vt_lds(buf), qf, acc, m, l, key0, my_pos, n_kv, c, qj, hf);
      }
      if (more) store_tile<D>(regs, ks_lds(buf ^ 1), vt_lds(buf ^ 1));
      __syncthreads();
    }

    // Epilogue: normalise, stage the wave's 32 x D output tile in LDS (the K^
    // tiles are no longer read), then store whole rows with 16-byte writes.
    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* ot = smem + wave * (kPrefillRowsPerWave * kOStride);
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 w;
        w.x = pack2(acc[t][4 * g4 + 0] * inv, acc[t][4 * g4 + 1] * inv);
        w.y = pack2(acc[t][4 * g4 + 2] * inv, acc[t][4 * g4 + 3] * inv);
        *reinterpret_cast<uint2*>(ot + qj * kOStride + 32 * t + 8 * g4 + 4 * hf) = w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (wave_active) {
      __bf16* obase = static_cast<__bf16*>(p.out);
#pragma unroll
      for (int i = 0; i < kPrefillRowsPerWave * (D / 8) / 64; ++i) {
        const int ci = lane + 64 * i;
        const int row = ci / (D / 8);
        const int c8 = ci % (D / 8);
        if (r0 + row < n_q)
          *reinterpret_cast<uint4*>(obase + ((q0 + r0 + row) * p.hq + h) * D + 8 * c8) =
              *reinterpret_cast<const uint4*>(ot + row * kOStride + 8 * c8);
      }
      if (hf == 0 && p.lse != nullptr && r0 + qj < n_q)
        p.lse[(int64_t)h * p.total_q + q0 + r0 + qj] =
            l_tot > 0.f ? (m + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    }
    __syncthreads();  // the output staging area is the next pass's K^ tile buffer
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnParams& p, int head_dim, int grid, hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(grid), dim3(kPrefillThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(grid), dim3(kPrefillThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace yoco
