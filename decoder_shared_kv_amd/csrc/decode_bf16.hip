// Decode split pass, bf16 storage, MFMA for both contractions.
//
// Every Cross-Decoder layer re-reads the whole shared cache once per decode
// step (page "YOCO", section "KV Cache 与计算量分析": repeated reads of the
// shared KV make its bandwidth the critical path), so this kernel is bound by
// HBM reads of K^ and V^. Design points:
//  * one workgroup = (share of the rows, KV head): the 128-row blocks of all
//    sequences are cut into equal shares, so the workgroups are balanced for
//    any mix of lengths; it reads each cache row of its share exactly once, for
//    ALL query heads of the KV group (<= 16 per workgroup), so GQA costs no
//    extra traffic;
//  * K^ rows go from HBM into MFMA A operands (16 B per lane), straight into
//    their operand layout or, with four or more KV heads, as whole rows
//    rearranged through a wave-private LDS tile:
//    S^T[key][head] = K^ . Q^T with v_mfma_f32_16x16x32_bf16, query heads padded
//    to 16 columns;
//  * the accumulator layout of S^T (lane = head, 4 consecutive keys per lane)
//    is exactly the B-operand layout of v_mfma_f32_16x16x16_bf16 over those
//    16 keys, so P^T never moves between lanes; V^ is transposed once through a
//    small wave-private LDS tile to become the A operand (V^T);
//  * online softmax in the base-2 domain, per lane, with two cross-lane max
//    reductions per iteration; the partial (max, sum, unnormalised O) of each
//    piece of a share is merged by decode_merge;
//  * nontemporal 16-byte loads: the cache is streamed once per call.
#include <hip/hip_bf16.h>

#include "internal.h"
#include "tile_common.h"

namespace yoco {

namespace {

// Tuning knobs (measured on MI355X at 8 x 131072, 4 x 131072, 16 x 17292 and
// 1 x 1048576 rows with the balanced split): one 16-key block per wave and
// iteration (1-4% ahead of two, three and four blocks are slower still), no
// register double buffer, nontemporal loads.
#ifndef YOCO_DEC_U
#define YOCO_DEC_U 1
#endif
#ifndef YOCO_DEC_PREFETCH
#define YOCO_DEC_PREFETCH 0
#endif
#ifndef YOCO_DEC_NT
#define YOCO_DEC_NT 1
#endif

constexpr int kDecWaves = 4;

// The cache is streamed once per call and is far larger than the 256 MB
// Infinity Cache: nontemporal loads keep it from evicting useful lines.
__device__ __forceinline__ uint4 stream_load16(const void* p) {
#if YOCO_DEC_NT
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}
__device__ __forceinline__ uint2 stream_load8(const void* p) {
#if YOCO_DEC_NT
  const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(t.x, t.y);
#else
  return *reinterpret_cast<const uint2*>(p);
#endif
}
constexpr int kVtStride = 20;  // 16 keys + 4 pad (bf16 elements) per transposed V^ row


__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

// Per-lane register tile of one iteration: U blocks of 16 keys. K^ and V^ are
// loaded alike, whole rows per instruction (16 lanes x D/16 dims cover one
// row, the 4 lane groups 4 consecutive rows): a probe of this load against
// the MFMA operand layout (64 bytes of each of 16 rows per instruction)
// measured 6.6-7.0 TB/s against 5.5-6.0. Both are then rearranged through a
// small wave-private LDS tile.
//
// Whole-row K^ loads pay an LDS round trip per block; they win with four or
// more KV heads (rows of one head 1 KB or more apart: +2-5%) and lose ~3% at
// two (1M rows, 16 x 2 heads), so KR = 1 is used from four KV heads on and the
// MFMA-layout loads (kd) below that.
template <int D, int U>
struct DecRegs {
  uint4 kd[U][D / 32];      // KR = 0: A operand of S^T, key (lane & 15), 8 dims at 32*kk + 8*(lane >> 4)
  uint32_t k[U][4][D / 32]; // KR = 1: keys 4*(lane >> 4) + i, dims (lane & 15) * D/16 .. +D/16 (as D/32 dwords)
  uint32_t v[U][4][D / 32]; // V^, whole rows as for KR = 1
};

template <int D, int U, int KR>
__device__ __forceinline__ void dec_load(DecRegs<D, U>& r, const __bf16* kbase, const __bf16* vbase,
                                         int64_t row_stride, int base, int last, int lane) {
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (KR) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int kkey = base + 16 * u + 4 * grp + i;
        kkey = kkey < last ? kkey : last;
        const int64_t off = (int64_t)kkey * row_stride + col * (D / 16);
        if constexpr (D == 128) {
          const uint4 x = stream_load16(kbase + off);
          r.k[u][i][0] = x.x; r.k[u][i][1] = x.y; r.k[u][i][2] = x.z; r.k[u][i][3] = x.w;
        } else {
          const uint2 x = stream_load8(kbase + off);
          r.k[u][i][0] = x.x; r.k[u][i][1] = x.y;
        }
      }
    } else {
      int key = base + 16 * u + col;
      key = key < last ? key : last;
      const __bf16* src = kbase + (int64_t)key * row_stride + 8 * grp;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) r.kd[u][kk] = stream_load16(src + 32 * kk);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int vkey = base + 16 * u + 4 * grp + i;
      vkey = vkey < last ? vkey : last;
      const __bf16* vs = vbase + (int64_t)vkey * row_stride + col * (D / 16);
      if constexpr (D == 128) {
        const uint4 x = stream_load16(vs);
        r.v[u][i][0] = x.x; r.v[u][i][1] = x.y; r.v[u][i][2] = x.z; r.v[u][i][3] = x.w;
      } else {
        const uint2 x = stream_load8(vs);
        r.v[u][i][0] = x.x; r.v[u][i][1] = x.y;
      }
    }
  }
}

// LDS: per-wave transposed V^ tiles; reused for the cross-wave combine at the end
template <int D, int U, int KR>
struct DecLds {
  static constexpr int kVtBytes = kDecWaves * U * D * kVtStride * 2;
  static constexpr int kKtBytes = KR ? kDecWaves * U * 16 * D * 2 : 0;   // row-major K^ blocks, after the V^T tiles
  static constexpr int kCombBytes = kDecWaves * 16 * (D + 2) * 4;
  static constexpr int kBytes = kVtBytes + kKtBytes > kCombBytes ? kVtBytes + kKtBytes : kCombBytes;
};

// K^ block in LDS: 16 rows of D/8 16-byte chunks, chunk c of row r stored at
// c ^ (r mod D/8), so that both the whole-row writes and the operand reads
// (16 rows x 4 chunks per instruction) spread over all banks.
template <int D>
__device__ __forceinline__ int kt_chunk(int r, int c) {
  return c ^ (r & (D / 8 - 1));
}

// Rows j0 .. j1-1 of sequence b (cache rows from `start`), all query heads of
// KV head kh's chunk hc: leaves the partial (m, l, O) of every head in its
// slot (h * p.slots + slot).
template <int D, int U, int KR>
__device__ __forceinline__ void decode_piece(const AttnParams& p, char* lds, int b, int64_t start, int j0, int j1,
                                             int kh, int hc, int slot) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  __bf16* vt = reinterpret_cast<__bf16*>(lds) + wave * (U * D * kVtStride);
  char* kt = lds + DecLds<D, U, KR>::kVtBytes + wave * (U * 16 * D * 2);

  const int h0 = kh * p.group + hc * 16;
  const int nh = p.group - hc * 16 < 16 ? p.group - hc * 16 : 16;

  // Q^T as the B operand: head column `col`, dims 32*kk + 8*grp .. +8
  bf16x8 qf[D / 32];
  {
    const __bf16* qsrc = static_cast<const __bf16*>(p.q) + ((int64_t)b * p.hq + h0 + (col < nh ? col : 0)) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint4 x = *reinterpret_cast<const uint4*>(qsrc + 32 * kk);
      if (col >= nh) x = make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int64_t row_stride = (int64_t)p.hkv * D;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + start * row_stride + (int64_t)kh * D;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + start * row_stride + (int64_t)kh * D;

  f32x4 acc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max of the base-2 scores of head `col` (same on its 4 lanes)
  float l = 0.f;        // this lane's share of the running sum of weights

  constexpr int kStep = kDecWaves * U * 16;
  static_assert(kDecodeBlockRows % kStep == 0, "pieces start at an iteration boundary");
  int base = j0 + wave * U * 16;
  DecRegs<D, U> cur;
#if YOCO_DEC_PREFETCH
  if (base < j1) dec_load<D, U, KR>(cur, kbase, vbase, row_stride, base, j1 - 1, lane);
#endif
  for (; base < j1; base += kStep) {
#if YOCO_DEC_PREFETCH
    DecRegs<D, U> nxt;
    const bool more = base + kStep < j1;
    if (more) dec_load<D, U, KR>(nxt, kbase, vbase, row_stride, base + kStep, j1 - 1, lane);
#else
    dec_load<D, U, KR>(cur, kbase, vbase, row_stride, base, j1 - 1, lane);
#endif

    // S^T = K^ . Q^T, 16 keys x 16 heads per block
    f32x4 s[U];
    if constexpr (KR) {
      // K^ block -> wave-private LDS (row-major, swizzled chunks), then back as
      // the A operand: key (lane & 15), 8 dims at 32*kk + 8*(lane >> 4)
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * grp + i;
          char* row = kt + (u * 16 + r) * (D * 2);
          if constexpr (D == 128) {
            *reinterpret_cast<uint4*>(row + 16 * kt_chunk<D>(r, col)) =
                make_uint4(cur.k[u][i][0], cur.k[u][i][1], cur.k[u][i][2], cur.k[u][i][3]);
          } else {
            *reinterpret_cast<uint2*>(row + 16 * kt_chunk<D>(r, col >> 1) + 8 * (col & 1)) =
                make_uint2(cur.k[u][i][0], cur.k[u][i][1]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        const char* row = kt + (u * 16 + col) * (D * 2);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const uint4 a = *reinterpret_cast<const uint4*>(row + 16 * kt_chunk<D>(col, 4 * kk + grp));
          s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], s[u], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.kd[u][kk]), qf[kk], s[u], 0,
                                                         0, 0);
      }
    }
    // scale to base 2, mask rows past the piece's end, block max
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = base + 16 * u + 4 * grp + r;
        const float t = key < j1 ? s[u][r] * p.scale_log2 : -INFINITY;
        s[u][r] = t;
        mx = fmaxf(mx, t);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));   // (lane swaps without LDS measured slower here)
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    m = m_new;
    float psum = 0.f;
    s16x4 pf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float e[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[r] = exp2f(s[u][r] - m_use);
        psum += e[r];
      }
      const uint32_t w0 = pack2(e[0], e[1]);
      const uint32_t w1 = pack2(e[2], e[3]);
      pf[u] = s16x4{(short)lo16(w0), (short)hi16(w0), (short)lo16(w1), (short)hi16(w1)};
    }
    l = l * alpha + psum;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc[t] *= alpha;

    // V^ block -> wave-private LDS, transposed: vt[u][d][key]
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int w = 0; w < D / 32; ++w) {
        const uint32_t a0 = cur.v[u][0][w], a1 = cur.v[u][1][w], a2 = cur.v[u][2][w], a3 = cur.v[u][3][w];
        const int d = col * (D / 16) + 2 * w;
        uint2 even, odd;
        even.x = lo16(a0) | (lo16(a1) << 16);
        even.y = lo16(a2) | (lo16(a3) << 16);
        odd.x = hi16(a0) | (hi16(a1) << 16);
        odd.y = hi16(a2) | (hi16(a3) << 16);
        *reinterpret_cast<uint2*>(vt + (u * D + d) * kVtStride + 4 * grp) = even;
        *reinterpret_cast<uint2*>(vt + (u * D + d + 1) * kVtStride + 4 * grp) = odd;
      }
    }
    // the LDS tile is private to this wave: LDS executes a wave's accesses in
    // order, so only compiler reordering must be prevented here
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // O^T += V^T . P^T, 16 dims x 16 heads per tile, 16 keys per block
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const uint2 a = *reinterpret_cast<const uint2*>(vt + (u * D + 16 * t + col) * kVtStride + 4 * grp);
        const s16x4 av = s16x4{(short)lo16(a.x), (short)hi16(a.x), (short)lo16(a.y), (short)hi16(a.y)};
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pf[u], acc[t], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#if YOCO_DEC_PREFETCH
    if (more) cur = nxt;
#endif
  }

  // combine the four waves of this piece
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();  // every wave is done with its V^ tile before the LDS is reused
  float* wo = reinterpret_cast<float*>(lds);              // [wave][16 heads][D]
  float* wml = wo + kDecWaves * 16 * D;                   // [wave][16 heads][2]
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) wo[(wave * 16 + col) * D + 16 * t + 4 * grp + r] = acc[t][r];
  }
  if (grp == 0) {
    wml[(wave * 16 + col) * 2 + 0] = m;
    wml[(wave * 16 + col) * 2 + 1] = l;
  }
  __syncthreads();
  {
    const int hh = threadIdx.x >> 4;               // head of the chunk
    const int d0 = (threadIdx.x & 15) * (D / 16);  // D/16 dims per thread
    float mw[kDecWaves];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      mw[w] = wml[(w * 16 + hh) * 2];
      M = fmaxf(M, mw[w]);
    }
    float sc[kDecWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      sc[w] = M == -INFINITY ? 0.f : exp2f(mw[w] - M);
      L = fmaf(wml[(w * 16 + hh) * 2 + 1], sc[w], L);
    }
    if (hh < nh) {
      const int64_t ps = (int64_t)(h0 + hh) * p.slots + slot;
      float* po = p.part_o + ps * D + d0;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) o = fmaf(wo[(w * 16 + hh) * D + d0 + i], sc[w], o);
        po[i] = o;
      }
      if ((threadIdx.x & 15) == 0) {
        p.part_ml[2 * ps + 0] = M;
        p.part_ml[2 * ps + 1] = L;
      }
    }
  }
}

// Minimum workgroups per CU the register budget must allow (1: no limit; the
// kernel needs about 228 VGPRs, two workgroups per CU).
#ifndef YOCO_DEC_OCC
#define YOCO_DEC_OCC 1
#endif

// Balanced split-K: the 128-row blocks of all sequences, in sequence order, are
// cut into `parts` contiguous shares of (nearly) equal size, one per
// workgroup of each (KV head, head chunk) column, so every workgroup streams
// the same number of rows whatever the mix of lengths. A share can span
// several sequences: each piece of it leaves its own partial, in slot
// share + sequence (distinct for every piece of a column). The workgroup that
// holds a sequence's first block records where its pieces are for the merge.
template <int D, int U, int KR>
__global__ __launch_bounds__(256, YOCO_DEC_OCC) void decode_split_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds[DecLds<D, U, KR>::kBytes];
  const int share = blockIdx.x;
  const int kh = blockIdx.y / p.head_chunks;
  const int hc = blockIdx.y % p.head_chunks;
  const int lane = threadIdx.x & 63;

  // every wave counts the sequences' blocks (the same loads, cached) and finds
  // the sequence holding this share's first block: no LDS, no barrier. The
  // first 64 sequences' rows, first pool rows and prefix stay in registers.
  int64_t start0;
  const int32_t n0 = decode_rows(p, lane, &start0);
  const int u0 = decode_blocks(n0);
  const int incl0 = wave_incl_scan_i32(u0);
  int64_t total = __builtin_amdgcn_readlane(incl0, 63);
  for (int c0 = 64; c0 < p.batch; c0 += 64) {
    int64_t st;
    total += wave_sum_i32(decode_blocks(decode_rows(p, c0 + lane, &st)));
  }
  total = uniform_i64(total);
  const int parts = total < p.splits ? (int)total : p.splits;
  if (share >= parts) return;
  const int64_t first = share_begin(share, total, parts);
  const int64_t last = share_begin(share + 1, total, parts);
  int b = p.batch;
  int64_t pre = total;
  int64_t carry = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 64) {
    int64_t st;
    const int u = c0 == 0 ? u0 : decode_blocks(decode_rows(p, c0 + lane, &st));
    const int incl = c0 == 0 ? incl0 : wave_incl_scan_i32(u);
    const int64_t before = carry + incl - u;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(u > 0 && before <= first && first < before + u);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      b = c0 + l;
      pre = carry + __builtin_amdgcn_readlane(incl - u, l);
      break;
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  b = __builtin_amdgcn_readfirstlane(b);
  pre = uniform_i64(pre);

  for (; b < p.batch && pre < last; ++b) {
    int64_t start;
    int32_t n_kv;
    if (b < 64) {   // from the scan's registers
      n_kv = __builtin_amdgcn_readlane(n0, b);
      start = (int64_t)(((uint64_t)__builtin_amdgcn_readlane((uint32_t)((uint64_t)start0 >> 32), b) << 32) |
                        __builtin_amdgcn_readlane((uint32_t)start0, b));
    } else {
      n_kv = decode_rows(p, b, &start);
    }
    const int u = decode_blocks(n_kv);
    if (u > 0) {
      const int64_t lo = (first > pre ? first : pre) - pre;
      const int64_t hi = (last < pre + u ? last : pre + u) - pre;
      if (lo == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        const int64_t s_last = share_of_block(pre + u - 1, total, parts);
        p.decode_meta[2 * b + 0] = share + b;
        p.decode_meta[2 * b + 1] = (int32_t)(s_last - share + 1);
      }
      const int j1 = hi * kDecodeBlockRows < n_kv ? (int)(hi * kDecodeBlockRows) : n_kv;
      decode_piece<D, U, KR>(p, lds, b, start, (int)(lo * kDecodeBlockRows), j1, kh, hc, share + b);
      __syncthreads();  // the combine's LDS reads are done before the next piece's tiles
    }
    pre += u;
  }
}

}  // namespace

hipError_t launch_decode_split_bf16(const AttnParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)p.splits, (unsigned)(p.hkv * p.head_chunks));
  const bool krow = p.hkv >= 4;
  if (head_dim == 64) {
    if (krow) hipLaunchKernelGGL((decode_split_bf16_kernel<64, YOCO_DEC_U, 1>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_split_bf16_kernel<64, YOCO_DEC_U, 0>), grid, dim3(256), 0, stream, p);
  } else {
    if (krow) hipLaunchKernelGGL((decode_split_bf16_kernel<128, YOCO_DEC_U, 1>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_split_bf16_kernel<128, YOCO_DEC_U, 0>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace yoco
