// gemm_nvfp4.hip -- expert-streaming grouped GEMMs on NVFP4 weights at
// mid-sized batches (a few dozen routes per local expert), where GEMM1 and
// GEMM2 are bound by HBM bandwidth on the weight bytes, not by the MFMAs.
// Two modes, a template argument: NVFP4 activations (W4A4) and bf16
// activations (W4A16).
//
// Same computation as gemm.hip ("flashinfer.fused_moe.cute_dsl_fused_moe",
// Parameters: quant_mode, fc2_input_scale; "vllm.models.flint.ops.moe_cute",
// module docstring):
//   GEMM1: y1 = act(alpha1[e] * x W1[e]^T) for the routes of expert e, y1
//          rounded once to bf16 (W4A4: then requantised to NVFP4 with
//          fc2_input_scale);
//   GEMM2: y2 = alpha2[e] * y1 W2[e]^T, stored as bf16 rows or weighted and
//          added into out with packed-bf16 atomics.
//
// Organisation, for bandwidth:
//  - a workgroup of 8 wavefronts owns one local expert, a block of 256
//    weight rows (GEMM1: 128 gate rows and their 128 up rows; GEMM2: 256
//    output columns) and the expert's routes, 48 (W4A4) or 32 (W4A16) at a
//    time; with the usual one pass per expert, each weight byte leaves HBM
//    once per forward and the tile padding of the plan costs nothing (the
//    kernel walks expert_offsets / expert_counts).
//  - each wavefront streams its 32 weight rows straight into registers, K
//    256 at a time through a ring of three register steps (two steps of
//    loads in flight while one is consumed), and decodes them right before
//    the MFMA.  W4A4: one v_cvt_scalef32_pk_f16_fp4 turns two E2M1 codes
//    into f16 (its scale operand takes only a power of two) and one
//    v_pk_mul_f16 applies the E4M3 block scale.  An E2M1 value times an E4M3
//    value has at most 6 significant bits and lies in [2^-10, 2688], so the
//    f16 operands are exact and v_mfma_f32_16x16x32_f16 (fp32 accumulation)
//    forms the same products as a bf16 MFMA would.  W4A16: the codes go to
//    fp32, take the scale in fp32 and are packed to bf16 (exact as well) for
//    v_mfma_f32_16x16x32_bf16.  128 VGPRs per lane: four wavefronts per
//    SIMD, two workgroups per CU.
//  - the routes' activations (x rows gathered by token for GEMM1, y1 slot rows
//    for GEMM2) go once per workgroup into a double-buffered LDS step that
//    the 8 wavefronts share: W4A4 decodes them to f16 the same way, W4A16
//    copies the bf16 rows.
//  - lane (r = lane%16, q = lane/16) of an MFMA holds weight row r of its
//    16-row n-tile and K [64q, 64q+64) of each step, walked in 8 sub-steps;
//    the activation rows in LDS hold the same K order, rows 16 bytes longer
//    than their data so that the operand reads are bank-conflict free.
//  - workgroups are dealt to the XCDs in runs of consecutive (expert, block)
//    items, so one expert's activation rows are read from one L2.
// Requirements (else another kernel runs): K (H for GEMM1, I for GEMM2) a
// multiple of 256; 16-byte aligned code arrays and row strides, 4-byte
// aligned scales.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace moe {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr int NV_THREADS = 512;
constexpr int NV_RB = 48;                     // W4A4: route rows per pass (3 MFMA m-tiles)
constexpr int NV_RB16 = 32;                   // W4A16: route rows per pass (2 MFMA m-tiles)
constexpr int NV_NB = 256;                    // weight rows per workgroup (32 per wavefront)
constexpr int NV_PAIRS = NV_NB / 2;           // GEMM1: gate / up pairs per workgroup
constexpr int NV_KS = 256;                    // K per step
constexpr int NV_ROW = NV_KS * 2 + 16;        // LDS row stride of the decoded activations (16 B pad)

struct NvArgs {
  const uint8_t* A;      // activation codes: x rows (GEMM1, by token) or y1 rows (GEMM2, by slot)
  const uint8_t* A_sf;   // their E4M3 block-16 scales
  int64_t a_row_bytes;
  int64_t a_sf_row;
  const uint8_t* W;
  const uint8_t* W_sf;
  const float* alpha;
  const float* alpha_up;  // GEMM1: the up half's scale (NULL: alpha)
  const float* pts;       // GEMM1: per-token input scale (NULL: none)
  const float* bias;      // NULL, or fp32 [E, 2 IP] (GEMM1: gate then up) / [E, H] (GEMM2)
  int K;
  int rows_per_expert;    // 2 IP (GEMM1) or H (GEMM2)
  int IP;                 // GEMM1: gate / up split (pairs)
  int n_out;              // y1 columns (GEMM1) or H (GEMM2)
  int n_blocks;           // weight-row blocks per expert
  const int32_t* p2e;
  const int32_t* offsets;
  const int32_t* counts;
  int El, top_k;
  GateAct act;
  const float* fc2_scale;
  void* Y;                // y1 codes (GEMM1) or y2 bf16 rows (GEMM2)
  uint8_t* Y_sf;
  const float* topk_w;
  float rsf;
  uint16_t* out;          // GEMM2 atomic finalize
  unsigned* amax;         // GEMM1 calibration: fp32 bits of the largest |y1|; nothing stored
};

// eight E2M1 codes (one dword, element 0 in the low nibble) times an f16
// block scale, as eight f16 (exact, see above)
DEV f16x8_t e2m1x8_f16(uint32_t w, _Float16 s) {
  f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// four E4M3 scale bytes (one dword) as four f16 values (exact: E4M3 values
// lie in [2^-9, 448])
struct Sc4 {
  f16x2_t lo, hi;
  DEV _Float16 operator[](int i) const { return i < 2 ? lo[i] : hi[i - 2]; }
};
DEV Sc4 e4m3x4_f16(uint32_t s) {
  return Sc4{__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false),
             __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true)};
}

// a 32-bit offset the compiler must keep 32-bit (so the loads take the
// scalar-base + 32-bit vector-offset form)
DEV uint32_t ou(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
// a value the compiler cannot see through (keeps derived values from being
// hoisted and held in registers across the K loop)
DEV int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// E4M3 byte i (0..3, a constant after unrolling) of a dword as fp32
DEV float e4m3_byte(uint32_t w, int i) {
  switch (i) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

// one K step of this lane's weights: 2 n-tiles x 64 codes + 4 scale bytes
struct WStep {
  u32x4_t c[2][2];
  uint32_t s[2];
};
// the two modes this file serves (the values of MOE_QUANT_W4A16 / MOE_QUANT_W4A4)
enum { NV_W4A16 = 0, NV_W4A4 = 1 };

// one K step of this thread's activation part.  W4A4: 32 codes + 2 scale
// bytes of one row; W4A16: three 16-byte chunks of bf16 (rows of their own)
template <int MODE> struct AStep;
template <> struct AStep<NV_W4A4> {
  u32x4_t c;
  uint32_t s;
};
// W4A16: 16-byte chunks of one bf16 activation step per thread
constexpr int NV_A16_PER = NV_RB16 * NV_KS * 2 / 16 / NV_THREADS;
template <> struct AStep<NV_W4A16> {
  u32x4_t c[NV_A16_PER];
};
// route rows per pass: W4A16 holds its activation step in registers as bf16
// (twice the bytes of NVFP4) and decodes weights through fp32, so its passes
// are 32 rows tall to stay within 128 VGPRs without spilling
template <int MODE> constexpr int nv_rb() { return MODE == NV_W4A16 ? NV_RB16 : NV_RB; }

// AK: the FC1 activation (ACT_*), fixed per instantiation so that the
// unrolled epilogue carries one kind's code
template <int MODE, int GEMM, bool ATOMIC, int AK>
__global__ __launch_bounds__(NV_THREADS, 4) void nvfp4_stream_kernel(const NvArgs a) {
  // MFMA operands: f16 (W4A4, both sides decoded exactly) or bf16 (W4A16)
  using op_t = std::conditional_t<MODE == NV_W4A4, f16x8_t, bf16x8_t>;
  constexpr int RB = nv_rb<MODE>();
  constexpr int BUF = RB * NV_ROW;  // one LDS activation step
  __shared__ __attribute__((aligned(16))) uint8_t xs[2 * BUF];
  __shared__ int32_t row_src[RB];
  __shared__ int32_t row_route[RB];

  // (expert, block) item of this workgroup: XCD x (blocks are dealt to the
  // 8 XCDs round-robin) takes items x*per .. x*per + per - 1
  const int per = gridDim.x >> 3;
  const int item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (item >= a.El * a.n_blocks) return;
  const int e = item / a.n_blocks;
  const int nb = item - e * a.n_blocks;
  const int cnt = a.counts[e];
  if (cnt <= 0) return;
  const int slot_base = a.offsets[e];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;

  // this lane's weight rows, one per n-tile.  GEMM1: n-tile 0 holds gate
  // rows and n-tile 1 the matching up rows, so a gate / up pair meets in one
  // lane; rows past the end of N (a partial block) load the last row and
  // their outputs are not stored.  Offsets are 32-bit from the expert's base
  // (one expert's weights stay below 4 GiB).
  const uint8_t* wbase = a.W + (int64_t)e * a.rows_per_expert * (a.K / 2);
  const uint8_t* sbase = a.W_sf + (int64_t)e * a.rows_per_expert * (a.K / 16);
  uint32_t wo[2], so[2];
#pragma unroll
  for (int n = 0; n < 2; n++) {
    int row;
    if constexpr (GEMM == 1) {
      const int j = min(nb * NV_PAIRS + wave * 16 + r, a.IP - 1);
      row = n * a.IP + j;
    } else {
      row = min(nb * NV_NB + wave * 32 + n * 16 + r, a.n_out - 1);
    }
    wo[n] = (uint32_t)row * (uint32_t)(a.K / 2) + 32u * q;
    so[n] = (uint32_t)row * (uint32_t)(a.K / 16) + 4u * q;
  }
  auto load_w = [&](WStep& b, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < 2; n++) {
      const uint32_t o = ou(wo[n] + (uint32_t)s * (NV_KS / 2));
      b.c[n][0] = *reinterpret_cast<const u32x4_t*>(wbase + o);
      b.c[n][1] = *reinterpret_cast<const u32x4_t*>(wbase + o + 16);
      b.s[n] = *reinterpret_cast<const uint32_t*>(sbase + ou(so[n] + (uint32_t)s * (NV_KS / 16)));
    }
  };

  // activation staging: thread (row ar, part ap) decodes K [32 ap, 32 ap + 32)
  // of one row per step
  const int ar = tid >> 3, ap = tid & 7;
  const int KT = a.K / NV_KS;

  for (int p0 = 0; p0 < cnt; p0 += RB) {
    const int valid = min(RB, cnt - p0);
    __syncthreads();  // the previous pass is done with the LDS steps and row tables
    if (tid < RB) {
      int route = -1, src = 0;
      if (tid < valid) {
        const int slot = slot_base + p0 + tid;
        route = a.p2e[slot];
        src = (GEMM == 1) ? route / a.top_k : slot;
      }
      row_src[tid] = src;
      row_route[tid] = route;
    }
    __syncthreads();

    // Activation staging.  Threads past the pass's rows load too: they read
    // row 0 of A, which exists, and store nothing, so each step issues the
    // same loads on every path.
    //  W4A4: thread (row ar, part ap) decodes K [32 ap, 32 ap + 32) of row ar;
    //  W4A16: thread tid copies chunks tid, tid + 512 of the step (chunk c:
    //  row c / 32, K [8 (c % 32), + 8)).
    constexpr int NA = MODE == NV_W4A4 ? 1 : NV_A16_PER;
    bool a_ok[NA];
    uint32_t aco[NA], aso = 0;
    if constexpr (MODE == NV_W4A4) {
      a_ok[0] = ar < valid;
      const int asrc = a_ok[0] ? row_src[ar] : 0;
      aco[0] = (uint32_t)asrc * (uint32_t)a.a_row_bytes + 16u * ap;
      aso = (uint32_t)asrc * (uint32_t)a.a_sf_row + 2u * ap;
    } else {
#pragma unroll
      for (int i = 0; i < NA; i++) {
        const int c = tid + NV_THREADS * i, row = c >> 5;
        a_ok[i] = row < valid;
        aco[i] = (uint32_t)(a_ok[i] ? row_src[row] : 0) * (uint32_t)a.a_row_bytes + 16u * (c & 31);
      }
    }
    auto load_a = [&](AStep<MODE>& b, int s) __attribute__((always_inline)) {
      if constexpr (MODE == NV_W4A4) {
        b.c = *reinterpret_cast<const u32x4_t*>(a.A + ou(aco[0] + (uint32_t)s * (NV_KS / 2)));
        b.s = *reinterpret_cast<const uint16_t*>(a.A_sf + ou(aso + (uint32_t)s * (NV_KS / 16)));
      } else {
#pragma unroll
        for (int i = 0; i < NA; i++)
          b.c[i] = *reinterpret_cast<const u32x4_t*>(a.A + ou(aco[i] + (uint32_t)s * (NV_KS * 2)));
      }
    };
    // into LDS step buffer `buf` (rows NV_ROW bytes apart, K in order)
    auto store_a = [&](const AStep<MODE>& b, int buf) __attribute__((always_inline)) {
      if constexpr (MODE == NV_W4A4) {
        if (!a_ok[0]) return;
        const Sc4 sc = e4m3x4_f16(b.s);
        uint8_t* row = xs + buf * BUF + ar * NV_ROW + 64 * ap;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const f16x8_t v = e2m1x8_f16(b.c[j], sc[j >> 1]);
          *reinterpret_cast<f16x8_t*>(row + 16 * j) = v;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NA; i++) {
          const int c = tid + NV_THREADS * i;
          if (a_ok[i]) *reinterpret_cast<u32x4_t*>(xs + buf * BUF + (c >> 5) * NV_ROW + 16 * (c & 31)) = b.c[i];
        }
      }
    };

    // the K loop and epilogue for MT 16-row m-tiles (MT = valid rows / 16, rounded up)
    auto run = [&](auto mt_c) __attribute__((always_inline)) {
      constexpr int MT = decltype(mt_c)::value;
      f32x4_t acc[MT][2];
#pragma unroll
      for (int m = 0; m < MT; m++)
#pragma unroll
        for (int n = 0; n < 2; n++) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      auto compute = [&](const WStep& w, int buf) __attribute__((always_inline)) {
        const uint8_t* xb = xs + buf * BUF + r * NV_ROW + 128 * q;
        Sc4 sc0, sc1;
        if constexpr (MODE == NV_W4A4) {
          sc0 = e4m3x4_f16(w.s[0]);
          sc1 = e4m3x4_f16(w.s[1]);
        }
#pragma unroll
        for (int j = 0; j < 8; j++) {
          op_t b0, b1;
          if constexpr (MODE == NV_W4A4) {
            b0 = e2m1x8_f16(w.c[0][j >> 2][j & 3], sc0[j >> 1]);
            b1 = e2m1x8_f16(w.c[1][j >> 2][j & 3], sc1[j >> 1]);
          } else {
            // E2M1 x E4M3 is exact in bf16 as well (two instructions per element)
            b0 = e2m1x8_scaled_to_bf16(w.c[0][j >> 2][j & 3], e4m3_byte(w.s[0], j >> 1));
            b1 = e2m1x8_scaled_to_bf16(w.c[1][j >> 2][j & 3], e4m3_byte(w.s[1], j >> 1));
          }
#pragma unroll
          for (int m = 0; m < MT; m++) {
            const op_t af = *reinterpret_cast<const op_t*>(xb + m * 16 * NV_ROW + 16 * j);
            if constexpr (MODE == NV_W4A4) {
              acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b0, acc[m][0], 0, 0, 0);
              acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b1, acc[m][1], 0, 0, 0);
            } else {
              acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b0, acc[m][0], 0, 0, 0);
              acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b1, acc[m][1], 0, 0, 0);
            }
          }
          // one sub-step's operands live at a time
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // three register steps in a ring: the loads of steps s+1 and s+2 are in
      // flight while step s is consumed.  Loads past the last step re-read
      // the last one, so every step issues the same loads.
      WStep w0, w1, w2;
      AStep<MODE> an;
      load_a(an, 0);
      load_w(w0, 0);
      load_w(w1, min(1, KT - 1));
      store_a(an, 0);
      __syncthreads();
      auto step = [&](const WStep& wc, WStep& wl, int s) __attribute__((always_inline)) {
        load_a(an, min(s + 1, KT - 1));
        load_w(wl, min(s + 2, KT - 1));
        compute(wc, s & 1);
        if (s + 1 < KT) store_a(an, (s + 1) & 1);
        __syncthreads();
      };
      int s = 0;
      for (; s + 3 <= KT; s += 3) {
        step(w0, w2, s);
        step(w1, w0, s + 1);
        step(w2, w1, s + 2);
      }
      if (s < KT) step(w0, w2, s);
      if (s + 1 < KT) step(w1, w0, s + 1);

      // ---- epilogue.  Lane holds rows 16 m + 4 q + i, column r of each n-tile.
      // The lane indices are re-derived through an opaque copy so that no
      // epilogue address is computed ahead of the K loop and held across it.
      const int lane = opaque(tid & 63), wave = opaque(tid >> 6);
      const int r = lane & 15, q = lane >> 4;
      const float alpha = a.alpha[e];
      if constexpr (GEMM == 1) {
        const float alpha_u = a.alpha_up ? a.alpha_up[e] : alpha;
        constexpr bool two = AK == ACT_RELU2;
        const float gs = a.amax ? 0.0f : *a.fc2_scale;
        uint8_t* Yq = reinterpret_cast<uint8_t*>(a.Y);
        const int col = nb * NV_PAIRS + wave * 16 + r;  // pair index
        const bool col_ok = col < a.IP;
        float mx = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; m++) {
          float y[2][4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = m * 16 + 4 * q + i;
            float g = acc[m][0][i] * alpha;
            float u = acc[m][1][i] * alpha_u;
            if (a.pts) {
              const float ps = (row < valid) ? a.pts[row_src[row]] : 1.0f;
              g = g * ps;
              u = u * ps;
            }
            if (a.bias && col_ok) {
              g = g + a.bias[(int64_t)e * 2 * a.IP + col];
              u = u + a.bias[(int64_t)e * 2 * a.IP + a.IP + col];
            }
            // y1 is rounded once to bf16; requantisation starts from that value
            if constexpr (two) {
              y[0][i] = bf16_to_f32(f32_to_bf16(relu2_f32(g)));
              y[1][i] = bf16_to_f32(f32_to_bf16(relu2_f32(u)));
            } else {
              y[0][i] = bf16_to_f32(f32_to_bf16(gated_act_k<AK>(g, u, a.act)));
              y[1][i] = 0.0f;
            }
            if (row < valid && col_ok) {
              mx = fmaxf(mx, fabsf(y[0][i]));
              if (two) mx = fmaxf(mx, fabsf(y[1][i]));
            }
          }
          if constexpr (MODE == NV_W4A16) {
            uint16_t* Y = reinterpret_cast<uint16_t*>(a.Y);
#pragma unroll
            for (int h = 0; h < (two ? 2 : 1); h++)
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const int row = m * 16 + 4 * q + i;
                if (row < valid && col_ok)
                  Y[(int64_t)(slot_base + p0 + row) * a.n_out + col + h * a.IP] = f32_to_bf16(y[h][i]);
              }
            continue;
          }
          if (a.amax) continue;
          // NVFP4 with the global scale fc2_input_scale; a block is the 16
          // columns of this wave's pairs (the 16 lanes of one lane group).
          // The pair count is a multiple of 16, so a block is valid as a whole.
#pragma unroll
          for (int h = 0; h < (two ? 2 : 1); h++) {
            const int cx = col + h * a.IP;
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int row = m * 16 + 4 * q + i;
              const float v = y[h][i];
              const float bamax = warp_max16(fabsf(v));
              const uint32_t sc = nvfp4_scale_code(bamax, gs);
              const uint32_t code = nvfp4_elem_code(v, e4m3_to_f32(sc), gs);
              const uint32_t other = __shfl_xor(code, 1);
              if (row < valid && col_ok) {
                const int64_t slot = slot_base + p0 + row;
                if ((r & 1) == 0) Yq[slot * (a.n_out / 2) + cx / 2] = (uint8_t)(code | (other << 4));
                if (r == 0) a.Y_sf[slot * (a.n_out / 16) + cx / 16] = (uint8_t)sc;
              }
            }
          }
        }
        if (a.amax) {
          // calibration pass: non-negative floats order like their bit patterns
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
          if (lane == 0 && mx > 0.0f) atomicMax(a.amax, __float_as_uint(mx));
        }
      } else {
#pragma unroll
        for (int m = 0; m < MT; m++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = m * 16 + 4 * q + i;
            const int64_t slot = slot_base + p0 + row;
            if constexpr (!ATOMIC) {
              uint16_t* Y = reinterpret_cast<uint16_t*>(a.Y);
              if (row < valid) {
#pragma unroll
                for (int n = 0; n < 2; n++) {
                  const int col = nb * NV_NB + wave * 32 + n * 16 + r;
                  if (col >= a.n_out) continue;  // past the end of a partial block
                  float v = acc[m][n][i] * alpha;
                  if (a.bias) v = v + a.bias[(int64_t)e * a.n_out + col];
                  Y[slot * a.n_out + col] = f32_to_bf16(v);
                }
              }
            } else {
              const int32_t route = (row < valid) ? row_route[row] : -1;
              const float wf = (route >= 0) ? __fmul_rn(a.topk_w[route], a.rsf) : 0.0f;
#pragma unroll
              for (int n = 0; n < 2; n++) {
                const int col = nb * NV_NB + wave * 32 + n * 16 + r;
                const bool ok = col < a.n_out;  // a partial block ends at an even column
                float v = acc[m][n][i] * alpha;
                if (a.bias && ok) v = v + a.bias[(int64_t)e * a.n_out + col];
                const float y2 = bf16_to_f32(f32_to_bf16(v));
                const float c = __fmul_rn(wf, y2);
                const float cn = __shfl_xor(c, 1);
                if (route >= 0 && ok && (r & 1) == 0) {
                  const int64_t t = route / a.top_k;
                  bf16x2_t pv = {(__bf16)c, (__bf16)cn};
                  __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<bf16x2_t*>(a.out + t * a.n_out + col),
                                                             pv);
                }
              }
            }
          }
      }
    };

    const int mt = (valid + 15) >> 4;
    if (mt == 1) {
      run(std::integral_constant<int, 1>{});
    } else if constexpr (RB == 32) {
      run(std::integral_constant<int, 2>{});
    } else {
      if (mt == 2) run(std::integral_constant<int, 2>{});
      else run(std::integral_constant<int, 3>{});
    }
  }
}

// ---------------------------------------------------------------- host side

static bool al(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

static bool nv_common(int mode, const moe_plan_t* plan, int K) {
  return (mode == MOE_QUANT_W4A4 || mode == MOE_QUANT_W4A16) && plan->tile <= 64 && K % NV_KS == 0 && K > 0;
}

bool nv_supported1(const Gemm1Params& p) {
  if (!nv_common(p.mode, p.plan, p.H) || !al(p.w1, 16) || !al(p.w1_sf, 4) || gemm1_pairs(p) % 16 != 0) return false;
  if (p.mode == MOE_QUANT_W4A4) {
    const int64_t stride = p.x_row_stride ? p.x_row_stride : p.H / 2;
    return stride % 16 == 0 && al(p.x, 16) && al(p.x_sf, 4);
  }
  const int64_t stride = p.x_row_stride ? p.x_row_stride : p.H;  // bf16 elements
  return stride % 8 == 0 && al(p.x, 16);
}

bool nv_supported2(const Gemm2Params& p) {
  if (!nv_common(p.mode, p.plan, p.I) || !al(p.y1, 16) || !al(p.w2, 16) || !al(p.w2_sf, 4)) return false;
  return p.mode == MOE_QUANT_W4A16 || al(p.y1_sf, 4);
}

static void nv_plan(NvArgs& a, const moe_plan_t* plan) {
  a.p2e = plan->permuted_to_expanded;
  a.offsets = plan->expert_offsets;
  a.counts = plan->expert_counts;
  a.El = plan->num_local_experts;
  a.top_k = plan->top_k;
}

template <int MODE, int GEMM, bool ATOMIC, int AK>
static hipError_t nv_launch(const NvArgs& a, hipStream_t stream) {
  const int items = a.El * a.n_blocks;
  if (items == 0) return hipSuccess;
  const int grid = (items + 7) / 8 * 8;
  nvfp4_stream_kernel<MODE, GEMM, ATOMIC, AK><<<grid, NV_THREADS, 0, stream>>>(a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t nv_launch1(const NvArgs& a, hipStream_t stream) {
  switch (a.act.kind) {
    case ACT_GEGLU_TANH: return nv_launch<MODE, 1, false, ACT_GEGLU_TANH>(a, stream);
    case ACT_SITU: return nv_launch<MODE, 1, false, ACT_SITU>(a, stream);
    case ACT_RELU2: return nv_launch<MODE, 1, false, ACT_RELU2>(a, stream);
    default: return nv_launch<MODE, 1, false, ACT_SWIGLU>(a, stream);
  }
}

static NvArgs nv_gemm1_args(const Gemm1Params& p) {
  NvArgs a = {};
  nv_plan(a, p.plan);
  a.A = reinterpret_cast<const uint8_t*>(p.x);
  a.A_sf = p.x_sf;
  if (p.mode == MOE_QUANT_W4A4) {
    a.a_row_bytes = p.x_row_stride ? p.x_row_stride : p.H / 2;
    a.a_sf_row = p.H / 16;
  } else {
    a.a_row_bytes = (p.x_row_stride ? p.x_row_stride : p.H) * 2;
  }
  a.W = p.w1;
  a.W_sf = p.w1_sf;
  a.alpha = p.w1_alpha;
  a.alpha_up = p.w1_alpha_up;
  a.pts = p.per_token_scale;
  a.bias = p.fc1_bias;
  a.K = p.H;
  a.IP = gemm1_pairs(p);
  a.rows_per_expert = 2 * a.IP;
  a.n_out = p.I;
  a.n_blocks = (a.IP + NV_PAIRS - 1) / NV_PAIRS;
  a.act = p.act;
  a.fc2_scale = p.fc2_input_scale;
  a.Y = p.y1;
  a.Y_sf = p.y1_sf;
  return a;
}

hipError_t launch_gemm1_nv(const Gemm1Params& p, hipStream_t stream) {
  if (p.mode == MOE_QUANT_W4A4) return nv_launch1<NV_W4A4>(nv_gemm1_args(p), stream);
  return nv_launch1<NV_W4A16>(nv_gemm1_args(p), stream);
}

hipError_t launch_gemm1_nv_amax(const Gemm1Params& p, unsigned* amax, hipStream_t stream) {
  NvArgs a = nv_gemm1_args(p);
  a.amax = amax;
  return nv_launch1<NV_W4A4>(a, stream);  // the calibration pass exists for W4A4 only
}

hipError_t launch_gemm2_nv(const Gemm2Params& p, hipStream_t stream) {
  NvArgs a = {};
  nv_plan(a, p.plan);
  a.A = reinterpret_cast<const uint8_t*>(p.y1);
  a.A_sf = p.y1_sf;
  a.a_row_bytes = p.mode == MOE_QUANT_W4A4 ? p.I / 2 : (int64_t)p.I * 2;
  a.a_sf_row = p.I / 16;
  a.W = p.w2;
  a.W_sf = p.w2_sf;
  a.alpha = p.w2_alpha;
  a.bias = p.fc2_bias;
  a.K = p.I;
  a.rows_per_expert = p.H;
  a.IP = p.I;
  a.n_out = p.H;
  a.n_blocks = (p.H + NV_NB - 1) / NV_NB;
  a.Y = p.y2;
  a.topk_w = p.topk_weights;
  a.rsf = p.routed_scaling_factor;
  a.out = p.out;
  if (p.mode == MOE_QUANT_W4A4) {
    if (p.out) return nv_launch<NV_W4A4, 2, true, ACT_SWIGLU>(a, stream);
    return nv_launch<NV_W4A4, 2, false, ACT_SWIGLU>(a, stream);
  }
  if (p.out) return nv_launch<NV_W4A16, 2, true, ACT_SWIGLU>(a, stream);
  return nv_launch<NV_W4A16, 2, false, ACT_SWIGLU>(a, stream);
}

}  // namespace moe
