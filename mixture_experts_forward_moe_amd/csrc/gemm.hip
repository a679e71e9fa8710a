// gemm.hip -- grouped GEMM1 (+ SwiGLU + requantisation) and GEMM2 (+ atomic
// finalize) of the fused MoE forward on gfx950 MFMA.
//
// The computation ("vllm.models.flint.ops.moe_cute", module docstring and
// grouped_moe; "flashinfer.fused_moe.cute_dsl_fused_moe", Parameters):
//   GEMM1: for each valid slot of expert e, y1 = SwiGLU(alpha1[e] * x[t] W1[e]^T)
//          with the weights' E2M1 x block-scale values exact in bf16, fp32
//          accumulation, gate/up kept in fp32 and y1 rounded once to bf16,
//          then requantised per mode (NVFP4 with fc2_input_scale, MXFP8).
//   GEMM2: y2 = alpha2[e] * y1 W2[e]^T, stored as bf16 rows (deterministic
//          finalize) or weighted and added into out with bf16 atomics.
//
// Kernel shape (one template for both GEMMs and all modes):
//  - a workgroup of 4 wavefronts owns BM permuted slots (inside one expert,
//    BM divides the plan tile) and 128 weight rows: for GEMM1 64 gate rows
//    j0.. and the 64 matching up rows I+j0.., so SwiGLU pairs sit in the
//    same lane; for GEMM2 128 output columns.
//  - K advances BK at a time through double-buffered LDS: activation rows
//    (gathered by token for GEMM1) and the packed weight tile, 16-byte
//    chunks XOR-swizzled by row so that both the global->LDS stores and the
//    MFMA operand reads are bank-conflict free.
//  - W4A16 / W4A4: v_mfma_f32_16x16x32_bf16.  Packed E2M1 weights stay 4-bit
//    in LDS; each lane decodes its 32 codes with the E4M3 block scale
//    (v_cvt_scalef32_pk_f32_fp4, one fp32 multiply, v_cvt_pk_bf16_f32) right
//    before the MFMA.  NVFP4 activations (W4A4) are decoded to bf16 once, on
//    their way into LDS.  Reduction order along K is free, so lane group q
//    takes K [32q, 32q+32) of each 128-wide step and walks it in 4 MFMAs.
//  - MXFP8_MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4 consumes E4M3 activations
//    and packed E2M1 weights with their E8M0 block-32 scales directly.
//  - Tile order: a flat grid, remapped so that each XCD (blocks are dealt
//    round-robin to the 8 XCDs) runs a contiguous range of tiles, slots
//    fastest, so the weight tile of one expert is re-read from its L2.
//  - Partial tiles (pull request 4440, description item 1: GEMM2 no longer
//    needs N to divide the tile): N (2I gate/up rows, or H) and K (H or I)
//    need only be multiples of 32.  Weight rows past N are clamped to the
//    last row for loading and their outputs are not stored; K past the end
//    of a step loads zero codes with zero scales, which add nothing.
#include "device_common.h"
#include "internal.h"

namespace moe {

enum { M_W4A16 = 0, M_W4A4 = 1, M_MX = 2 };

constexpr int GEMM_THREADS = 256;
constexpr int BN = 128;  // weight rows per workgroup

struct KArgs {
  const uint8_t* A;     // activations: x (GEMM1) or y1 (GEMM2)
  const uint8_t* A_sf;  // their block scales (W4A4, MX)
  int64_t a_row_bytes;  // row stride of A in bytes
  int64_t a_sf_row;     // row stride of A_sf in bytes
  const uint8_t* W;
  const uint8_t* W_sf;
  const float* alpha;
  const float* alpha_up;  // GEMM1: the up half's scale (NULL: alpha)
  const float* pts;       // GEMM1, W4A4: per-token input row scale (NULL: none)
  const float* bias;      // NULL, or fp32 [E, 2I] (GEMM1: gate then up) / [E, H] (GEMM2)
  int K;                // contraction length (H for GEMM1, I for GEMM2)
  int rows_per_expert;  // 2I or H
  int I;                // GEMM1: gate/up split
  int n_out;            // output columns: I (GEMM1) or H (GEMM2)
  const int32_t* p2e;
  const int32_t* tile_expert;
  const int32_t* tile_limit;
  const int32_t* offsets;
  int El, tile, top_k;
  int m_tiles, n_tiles, total_tiles;
  GateAct act;          // FC1 activation
  const float* fc2_scale;
  void* Y;              // y1 codes / y1 bf16 / y2 bf16
  uint8_t* Y_sf;
  const float* topk_w;
  float rsf;
  uint16_t* out;        // atomic finalize
  unsigned* amax;       // GEMM1 calibration: fp32 bits of the largest |y1| (nothing stored); NULL otherwise
};

template <int MODE>
struct Cfg {
  static constexpr int BK = (MODE == M_MX) ? 256 : 128;
  static constexpr int A_CHUNKS = (MODE == M_MX) ? BK / 16 : BK * 2 / 16;  // 16-byte chunks per A row in LDS
  static constexpr int B_CHUNKS = BK / 2 / 16;                              // 16-byte chunks per weight row
};

// swizzled 16-byte chunk position inside an LDS tile of `rows` rows
DEV int sw(int kc, int row, int rows) { return kc * rows + (row ^ (kc & 7)); }

// the 8 block-scale bytes of one K step starting at p, of which only the
// first n (>= 1) lie inside the row: the rest read as 0 (a zero scale)
DEV uint2 load_scales8(const uint8_t* p, int n) {
  if (n >= 8) return *reinterpret_cast<const uint2*>(p);
  uint32_t w[2] = {0u, 0u};
  for (int i = 0; i < n; i++) w[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
  return make_uint2(w[0], w[1]);
}

template <int MODE, int GEMM, int BM, bool ATOMIC>
__global__ __launch_bounds__(GEMM_THREADS, 2) void grouped_gemm_kernel(const KArgs a) {
  using C = Cfg<MODE>;
  constexpr int BK = C::BK;
  constexpr int AC = C::A_CHUNKS;
  constexpr int BC = C::B_CHUNKS;
  constexpr int MT = BM / 16;
  constexpr int A_BYTES = BM * AC * 16;
  constexpr int B_BYTES = BN * BC * 16;
  constexpr int BSF_BYTES = BN * 8;
  constexpr int ASF_BYTES = (MODE == M_MX) ? BM * 8 : 0;
  constexpr int STAGE = A_BYTES + B_BYTES + BSF_BYTES + ASF_BYTES;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int64_t row_src[BM];
  __shared__ int32_t row_route[BM];
  __shared__ float red[4][BM];

  // ---- tile of this workgroup (XCD-aware: XCD x runs logical tiles x*per ..)
  const int G = gridDim.x;
  const int per = G >> 3;
  const int L = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (L >= a.total_tiles) return;
  const int m_tile = L % a.m_tiles;
  const int n_tile = L / a.m_tiles;
  const int slot0 = m_tile * BM;
  if (slot0 >= a.offsets[a.El]) return;
  const int pt = slot0 / a.tile;
  const int e = a.tile_expert[pt];
  const int lim = a.tile_limit[pt];
  if (e < 0 || lim <= slot0) return;
  const int valid = min(BM, lim - slot0);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;

  for (int i = tid; i < BM; i += GEMM_THREADS) {
    int64_t src = -1;
    int32_t route = -1;
    if (i < valid) {
      route = a.p2e[slot0 + i];
      const int64_t row = (GEMM == 1) ? (int64_t)(route / a.top_k) : (int64_t)(slot0 + i);
      src = row;
    }
    row_src[i] = src;
    row_route[i] = route;
  }
  __syncthreads();

  // weight rows of this tile
  const int j0 = n_tile * 64;   // GEMM1: gate/up column block
  const int n0 = n_tile * BN;   // GEMM2: output column block
  // rows past the end of N (a partial last tile) load the last row; their
  // outputs are never stored
  auto wrow = [&](int lr) -> int64_t {
    int n = (GEMM == 1) ? (lr < 64 ? min(j0 + lr, a.I - 1) : a.I + min(j0 + lr - 64, a.I - 1))
                        : min(n0 + lr, a.n_out - 1);
    return (int64_t)e * a.rows_per_expert + n;
  };
  const int64_t w_row_bytes = a.K / 2;
  const int64_t w_sf_row = (MODE == M_MX) ? a.K / 32 : a.K / 16;

  // ---- per-thread global prefetch registers
  constexpr int A_LOADS = (MODE == M_W4A4) ? (BM * (BK / 32) + GEMM_THREADS - 1) / GEMM_THREADS
                                           : (BM * AC + GEMM_THREADS - 1) / GEMM_THREADS;
  constexpr int B_LOADS = (BN * BC) / GEMM_THREADS;
  u32x4_t ra[A_LOADS];
  uint32_t ra_sf[A_LOADS];
  u32x4_t rb[B_LOADS];
  uint2 rbsf = make_uint2(0u, 0u);
  uint2 rasf = make_uint2(0u, 0u);

  auto load_global = [&](int k0) {
    // activations
    if constexpr (MODE == M_W4A4) {
      // BM rows x (BK/32) packed chunks of 32 codes, plus their 2 scale bytes
#pragma unroll
      for (int i = 0; i < A_LOADS; i++) {
        int c = tid + i * GEMM_THREADS;
        int row = c / (BK / 32), part = c % (BK / 32);
        ra[i] = u32x4_t{0u, 0u, 0u, 0u};
        ra_sf[i] = 0u;
        if (row < BM && row < valid && k0 + 32 * part < a.K) {
          int64_t src = row_src[row];
          const uint8_t* p = a.A + src * a.a_row_bytes + k0 / 2 + part * 16;
          ra[i] = *reinterpret_cast<const u32x4_t*>(p);
          const uint8_t* s = a.A_sf + src * a.a_sf_row + k0 / 16 + part * 2;
          ra_sf[i] = *reinterpret_cast<const uint16_t*>(s);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_LOADS; i++) {
        int c = tid + i * GEMM_THREADS;
        int row = c / AC, kc = c % AC;
        ra[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (row < BM && row < valid && k0 + kc * (MODE == M_MX ? 16 : 8) < a.K) {
          int64_t src = row_src[row];
          const uint8_t* p = a.A + src * a.a_row_bytes + (MODE == M_MX ? k0 : k0 * 2) + kc * 16;
          ra[i] = *reinterpret_cast<const u32x4_t*>(p);
        }
      }
      if constexpr (MODE == M_MX) {
        if (tid < BM) {
          rasf = make_uint2(0u, 0u);
          if (tid < valid) rasf = load_scales8(a.A_sf + row_src[tid] * a.a_sf_row + k0 / 32, (a.K - k0) / 32);
        }
      }
    }
    // weights
#pragma unroll
    for (int i = 0; i < B_LOADS; i++) {
      int c = tid + i * GEMM_THREADS;
      int lr = c / BC, kc = c % BC;
      const uint8_t* p = a.W + wrow(lr) * w_row_bytes + k0 / 2 + kc * 16;
      rb[i] = (k0 + 32 * kc < a.K) ? *reinterpret_cast<const u32x4_t*>(p) : u32x4_t{0u, 0u, 0u, 0u};
    }
    if (tid < BN) {
      const int blk = (MODE == M_MX) ? 32 : 16;
      rbsf = load_scales8(a.W_sf + wrow(tid) * w_sf_row + k0 / blk, (a.K - k0) / blk);
    }
  };

  auto store_lds = [&](int buf) {
    uint8_t* st = smem + buf * STAGE;
    u32x4_t* As = reinterpret_cast<u32x4_t*>(st);
    u32x4_t* Bs = reinterpret_cast<u32x4_t*>(st + A_BYTES);
    uint2* Bsf = reinterpret_cast<uint2*>(st + A_BYTES + B_BYTES);
    if constexpr (MODE == M_W4A4) {
#pragma unroll
      for (int i = 0; i < A_LOADS; i++) {
        int c = tid + i * GEMM_THREADS;
        int row = c / (BK / 32), part = c % (BK / 32);
        if (row < BM) {
          float s0 = e4m3_to_f32(ra_sf[i] & 255u), s1 = e4m3_to_f32((ra_sf[i] >> 8) & 255u);
          As[sw(4 * part + 0, row, BM)] = __builtin_bit_cast(u32x4_t, e2m1x8_scaled_to_bf16(ra[i][0], s0));
          As[sw(4 * part + 1, row, BM)] = __builtin_bit_cast(u32x4_t, e2m1x8_scaled_to_bf16(ra[i][1], s0));
          As[sw(4 * part + 2, row, BM)] = __builtin_bit_cast(u32x4_t, e2m1x8_scaled_to_bf16(ra[i][2], s1));
          As[sw(4 * part + 3, row, BM)] = __builtin_bit_cast(u32x4_t, e2m1x8_scaled_to_bf16(ra[i][3], s1));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_LOADS; i++) {
        int c = tid + i * GEMM_THREADS;
        int row = c / AC, kc = c % AC;
        if (row < BM) As[sw(kc, row, BM)] = ra[i];
      }
      if constexpr (MODE == M_MX) {
        if (tid < BM) reinterpret_cast<uint2*>(st + A_BYTES + B_BYTES + BSF_BYTES)[tid] = rasf;
      }
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; i++) {
      int c = tid + i * GEMM_THREADS;
      int lr = c / BC, kc = c % BC;
      Bs[sw(kc, lr, BN)] = rb[i];
    }
    if (tid < BN) Bsf[tid] = rbsf;
  };

  // ---- accumulators: [row tile][col tile 0/1]
  f32x4_t acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; m++)
#pragma unroll
    for (int n = 0; n < 2; n++) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // local weight row of column tile n for this lane
  auto bcol = [&](int n) -> int {
    return (GEMM == 1) ? (n * 64 + wave * 16 + r16) : (wave * 32 + n * 16 + r16);
  };

  auto compute = [&](int buf) {
    const uint8_t* st = smem + buf * STAGE;
    const u32x4_t* As = reinterpret_cast<const u32x4_t*>(st);
    const u32x4_t* Bs = reinterpret_cast<const u32x4_t*>(st + A_BYTES);
    const uint8_t* Bsf = st + A_BYTES + B_BYTES;
    if constexpr (MODE == M_MX) {
      const uint8_t* Asf = st + A_BYTES + B_BYTES + BSF_BYTES;
#pragma unroll
      for (int s = 0; s < BK / 128; s++) {
        i32x8_t bf[2];
        int bsc[2];
#pragma unroll
        for (int n = 0; n < 2; n++) {
          int lr = bcol(n);
          u32x4_t b = Bs[sw(4 * s + q, lr, BN)];
          bf[n] = i32x8_t{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
          bsc[n] = Bsf[lr * 8 + 4 * s + q];
        }
#pragma unroll
        for (int m = 0; m < MT; m++) {
          int row = m * 16 + r16;
          u32x4_t a0 = As[sw(8 * s + q, row, BM)];
          u32x4_t a1 = As[sw(8 * s + 4 + q, row, BM)];
          i32x8_t af = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                               (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          int asc = Asf[row * 8 + 4 * s + q];
#pragma unroll
          for (int n = 0; n < 2; n++)
            acc[m][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[n], acc[m][n], 0, 4, 0, asc, 0,
                                                                         bsc[n]);
        }
      }
    } else {
      // lane group q owns K [32q, 32q+32) of this 128-wide step
      bf16x8_t bf[2][4];
#pragma unroll
      for (int n = 0; n < 2; n++) {
        int lr = bcol(n);
        u32x4_t b = Bs[sw(q, lr, BN)];
        uint32_t sc2 = *reinterpret_cast<const uint16_t*>(Bsf + lr * 8 + 2 * q);
        float s0 = e4m3_to_f32(sc2 & 255u), s1 = e4m3_to_f32(sc2 >> 8);
        bf[n][0] = e2m1x8_scaled_to_bf16(b[0], s0);
        bf[n][1] = e2m1x8_scaled_to_bf16(b[1], s0);
        bf[n][2] = e2m1x8_scaled_to_bf16(b[2], s1);
        bf[n][3] = e2m1x8_scaled_to_bf16(b[3], s1);
      }
#pragma unroll
      for (int s = 0; s < 4; s++) {
#pragma unroll
        for (int m = 0; m < MT; m++) {
          bf16x8_t af = __builtin_bit_cast(bf16x8_t, As[sw(4 * q + s, m * 16 + r16, BM)]);
#pragma unroll
          for (int n = 0; n < 2; n++)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[n][s], acc[m][n], 0, 0, 0);
        }
      }
    }
  };

  // ---- main loop
  const int KT = (a.K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < KT; kt++) {
    if (kt + 1 < KT) load_global((kt + 1) * BK);
    compute(kt & 1);
    if (kt + 1 < KT) store_lds((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue.  Lane holds rows m*16 + 4q + i, column r16 of each tile.
  const float alpha = a.alpha[e];
  if constexpr (GEMM == 1) {
    const float alpha_u = a.alpha_up ? a.alpha_up[e] : alpha;
    const int col = j0 + wave * 16 + r16;  // output column of y1 (pair index)
    const bool col_ok = col < a.I;           // false past the end of a partial tile
    // gated: one output per gate / up pair; ReLU^2 (non-gated): the two
    // rows of a pair are outputs col and a.I + col
    const bool two = a.act.kind == ACT_RELU2;
    float y[2][MT][4];
#pragma unroll
    for (int m = 0; m < MT; m++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float g = acc[m][0][i] * alpha;
        float u = acc[m][1][i] * alpha_u;
        if (a.pts) {
          const int row = m * 16 + 4 * q + i;
          const float s = (row < valid) ? a.pts[row_route[row] / a.top_k] : 1.0f;
          g = g * s;
          u = u * s;
        }
        if (a.bias && col_ok) {
          g = g + a.bias[(int64_t)e * 2 * a.I + col];
          u = u + a.bias[(int64_t)e * 2 * a.I + a.I + col];
        }
        // y1 is rounded once to bf16; requantisation starts from that value
        if (two) {
          y[0][m][i] = bf16_to_f32(f32_to_bf16(relu2_f32(g)));
          y[1][m][i] = bf16_to_f32(f32_to_bf16(relu2_f32(u)));
        } else {
          y[0][m][i] = bf16_to_f32(f32_to_bf16(gated_act_f32(g, u, a.act)));
          y[1][m][i] = 0.0f;
        }
      }
    if (a.amax) {
      // calibration pass: the largest |y1| over the valid rows and columns
      // (non-negative floats order like their bit patterns)
      float mx = 0.0f;
#pragma unroll
      for (int m = 0; m < MT; m++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int row = m * 16 + 4 * q + i;
          if (row < valid && col_ok) {
            mx = fmaxf(mx, fabsf(y[0][m][i]));
            if (two) mx = fmaxf(mx, fabsf(y[1][m][i]));
          }
        }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      if (lane == 0 && mx > 0.0f) atomicMax(a.amax, __float_as_uint(mx));
      return;
    }
    auto store = [&](const float (&ys)[MT][4], const int cx) __attribute__((always_inline)) {
      if constexpr (MODE == M_W4A16) {
        uint16_t* Y = reinterpret_cast<uint16_t*>(a.Y);
#pragma unroll
        for (int m = 0; m < MT; m++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            int row = m * 16 + 4 * q + i;
            if (row < valid && col_ok) Y[(int64_t)(slot0 + row) * a.n_out + cx] = f32_to_bf16(ys[m][i]);
          }
      } else if constexpr (MODE == M_W4A4) {
        // NVFP4 with the global scale fc2_input_scale; a block is the 16
        // columns of this wave's tile (the 16 lanes of one lane group)
        const float gs = *a.fc2_scale;
        uint8_t* Yq = reinterpret_cast<uint8_t*>(a.Y);
#pragma unroll
        for (int m = 0; m < MT; m++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            int row = m * 16 + 4 * q + i;
            float bamax = warp_max16(fabsf(ys[m][i]));
            uint32_t sc = nvfp4_scale_code(bamax, gs);
            uint32_t code = nvfp4_elem_code(ys[m][i], e4m3_to_f32(sc), gs);
            uint32_t other = __shfl_xor(code, 1);
            if (row < valid && col_ok) {
              int64_t slot = slot0 + row;
              if ((r16 & 1) == 0) Yq[slot * (a.n_out / 2) + cx / 2] = (uint8_t)(code | (other << 4));
              if (r16 == 0) a.Y_sf[slot * (a.n_out / 16) + cx / 16] = (uint8_t)sc;
            }
          }
      } else {
        // MXFP8: a block of 32 columns spans this wave and its neighbour
        __syncthreads();  // the previous set's exchange has been read
#pragma unroll
        for (int m = 0; m < MT; m++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            float am = warp_max16(fabsf(ys[m][i]));
            if (r16 == 0) red[wave][m * 16 + 4 * q + i] = am;
          }
        __syncthreads();
        uint8_t* Yq = reinterpret_cast<uint8_t*>(a.Y);
#pragma unroll
        for (int m = 0; m < MT; m++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            int row = m * 16 + 4 * q + i;
            float am = fmaxf(red[wave][row], red[wave ^ 1][row]);
            uint32_t code = mx_scale_code(am, 8);
            uint32_t b = f32x2_to_e4m3x2_mx(ys[m][i], 0.0f, code) & 255u;
            if (row < valid && col_ok) {
              int64_t slot = slot0 + row;
              Yq[slot * a.n_out + cx] = (uint8_t)b;
              if (r16 == 0 && (wave & 1) == 0) a.Y_sf[slot * (a.n_out / 32) + cx / 32] = (uint8_t)code;
            }
          }
      }
    };
    store(y[0], col);
    if (two) store(y[1], a.I + col);
  } else {
    // GEMM2: columns n0 + wave*32 + n*16 + r16
#pragma unroll
    for (int m = 0; m < MT; m++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int row = m * 16 + 4 * q + i;
        if constexpr (!ATOMIC) {
          uint16_t* Y = reinterpret_cast<uint16_t*>(a.Y);
          if (row < valid) {
#pragma unroll
            for (int n = 0; n < 2; n++) {
              int col = n0 + wave * 32 + n * 16 + r16;
              if (col >= a.n_out) continue;  // past the end of a partial tile
              float v = acc[m][n][i] * alpha;
              if (a.bias) v = v + a.bias[(int64_t)e * a.n_out + col];
              Y[(int64_t)(slot0 + row) * a.n_out + col] = f32_to_bf16(v);
            }
          }
        } else {
          int32_t route = (row < valid) ? row_route[row] : -1;
          float wf = (route >= 0) ? __fmul_rn(a.topk_w[route], a.rsf) : 0.0f;
#pragma unroll
          for (int n = 0; n < 2; n++) {
            int col = n0 + wave * 32 + n * 16 + r16;
            const bool ok = col < a.n_out;  // a partial tile ends at an even column
            float v = acc[m][n][i] * alpha;
            if (a.bias && ok) v = v + a.bias[(int64_t)e * a.n_out + col];
            float y2 = bf16_to_f32(f32_to_bf16(v));
            float c = __fmul_rn(wf, y2);
            float cn = __shfl_xor(c, 1);
            if (route >= 0 && ok && (r16 & 1) == 0) {
              int64_t t = route / a.top_k;
              bf16x2_t v = {(__bf16)c, (__bf16)cn};
              __builtin_amdgcn_global_atomic_fadd_v2bf16(
                  reinterpret_cast<bf16x2_t*>(a.out + t * a.n_out + col), v);
            }
          }
        }
      }
  }
}

// ---------------------------------------------------------------- host side

template <int MODE, int GEMM, int BM, bool ATOMIC>
static hipError_t launch_one(const KArgs& a, hipStream_t stream) {
  int grid = (a.total_tiles + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  grouped_gemm_kernel<MODE, GEMM, BM, ATOMIC><<<grid, GEMM_THREADS, 0, stream>>>(a);
  return hipGetLastError();
}

static int pick_bm(int tile) { return tile >= 64 ? 64 : (tile >= 32 ? 32 : 16); }

template <int GEMM, bool ATOMIC>
static hipError_t dispatch(int mode, int bm, const KArgs& a, hipStream_t s) {
#define MOE_CASE(MD, B) \
  if (mode == MD && bm == B) return launch_one<MD, GEMM, B, ATOMIC>(a, s);
  MOE_CASE(M_W4A16, 16) MOE_CASE(M_W4A16, 32) MOE_CASE(M_W4A16, 64)
  MOE_CASE(M_W4A4, 16) MOE_CASE(M_W4A4, 32) MOE_CASE(M_W4A4, 64)
  MOE_CASE(M_MX, 16) MOE_CASE(M_MX, 32) MOE_CASE(M_MX, 64)
#undef MOE_CASE
  return hipErrorInvalidValue;
}

static void plan_args(KArgs& a, const moe_plan_t* plan, int bm) {
  a.p2e = plan->permuted_to_expanded;
  a.tile_expert = plan->tile_to_expert;
  a.tile_limit = plan->tile_to_mn_limit;
  a.offsets = plan->expert_offsets;
  a.El = plan->num_local_experts;
  a.tile = plan->tile;
  a.top_k = plan->top_k;
  a.m_tiles = (int)(plan->route_slots / bm);
}

hipError_t launch_gemm1(const Gemm1Params& p, hipStream_t stream) {
  if (nv_supported1(p)) return launch_gemm1_nv(p, stream);
  if (wide_supported1(p)) return launch_gemm1_wide(p, stream);
  if (mxw_supported1(p)) return launch_gemm1_mxw(p, stream);
  if (mx_supported1(p)) return launch_gemm1_mx(p, stream);
  KArgs a = {};
  const int bm = pick_bm(p.plan->tile);
  plan_args(a, p.plan, bm);
  a.A = reinterpret_cast<const uint8_t*>(p.x);
  a.A_sf = p.x_sf;
  const int64_t stride = p.x_row_stride ? p.x_row_stride : (p.mode == M_W4A4 ? p.H / 2 : p.H);
  a.a_row_bytes = (p.mode == M_W4A16) ? stride * 2 : stride;
  a.a_sf_row = (p.mode == M_MX) ? p.H / 32 : p.H / 16;
  a.W = p.w1;
  a.W_sf = p.w1_sf;
  a.alpha = p.w1_alpha;
  a.alpha_up = p.w1_alpha_up;
  a.pts = p.per_token_scale;
  a.bias = p.fc1_bias;
  a.K = p.H;
  const int IP = gemm1_pairs(p);
  a.rows_per_expert = 2 * IP;
  a.I = IP;
  a.n_out = p.I;
  a.n_tiles = (IP + 63) / 64;
  a.total_tiles = a.m_tiles * a.n_tiles;
  a.act = p.act;
  a.fc2_scale = p.fc2_input_scale;
  a.Y = p.y1;
  a.Y_sf = p.y1_sf;
  return dispatch<1, false>(p.mode, bm, a, stream);
}

hipError_t launch_gemm1_amax(const Gemm1Params& p, unsigned* amax, hipStream_t stream) {
  if (nv_supported1(p)) return launch_gemm1_nv_amax(p, amax, stream);
  KArgs a = {};
  const int bm = pick_bm(p.plan->tile);
  plan_args(a, p.plan, bm);
  a.A = reinterpret_cast<const uint8_t*>(p.x);
  a.A_sf = p.x_sf;
  const int64_t stride = p.x_row_stride ? p.x_row_stride : (p.mode == M_W4A4 ? p.H / 2 : p.H);
  a.a_row_bytes = (p.mode == M_W4A16) ? stride * 2 : stride;
  a.a_sf_row = (p.mode == M_MX) ? p.H / 32 : p.H / 16;
  a.W = p.w1;
  a.W_sf = p.w1_sf;
  a.alpha = p.w1_alpha;
  a.alpha_up = p.w1_alpha_up;
  a.pts = p.per_token_scale;
  a.bias = p.fc1_bias;
  a.K = p.H;
  const int IP = gemm1_pairs(p);
  a.rows_per_expert = 2 * IP;
  a.I = IP;
  a.n_out = p.I;
  a.n_tiles = (IP + 63) / 64;
  a.total_tiles = a.m_tiles * a.n_tiles;
  a.act = p.act;
  a.amax = amax;
  return dispatch<1, false>(p.mode, bm, a, stream);
}

hipError_t launch_gemm2(const Gemm2Params& p, hipStream_t stream) {
  if (nv_supported2(p)) return launch_gemm2_nv(p, stream);
  if (wide_supported2(p)) return launch_gemm2_wide(p, stream);
  if (mxw_supported2(p)) return launch_gemm2_mxw(p, stream);
  if (mx_supported2(p)) return launch_gemm2_mx(p, stream);
  KArgs a = {};
  const int bm = pick_bm(p.plan->tile);
  plan_args(a, p.plan, bm);
  a.A = reinterpret_cast<const uint8_t*>(p.y1);
  a.A_sf = p.y1_sf;
  a.a_row_bytes = (p.mode == M_W4A16) ? (int64_t)p.I * 2 : (p.mode == M_W4A4 ? p.I / 2 : p.I);
  a.a_sf_row = (p.mode == M_MX) ? p.I / 32 : p.I / 16;
  a.W = p.w2;
  a.W_sf = p.w2_sf;
  a.alpha = p.w2_alpha;
  a.bias = p.fc2_bias;
  a.K = p.I;
  a.rows_per_expert = p.H;
  a.I = p.I;
  a.n_out = p.H;
  a.n_tiles = (p.H + BN - 1) / BN;
  a.total_tiles = a.m_tiles * a.n_tiles;
  a.Y = p.y2;
  a.topk_w = p.topk_weights;
  a.rsf = p.routed_scaling_factor;
  a.out = p.out;
  if (p.out) return dispatch<2, true>(p.mode, bm, a, stream);
  return dispatch<2, false>(p.mode, bm, a, stream);
}

}  // namespace moe
