// gfx950 kernels of libssmscan: the Mamba-2 (SSD) scan in chunked matrix form
// on MFMA, and its decode step.
//
// What is computed (pages: "Mamba и State Space Models", nareshka.ru, section
// "Mamba-2: State Space Duality": A is one scalar per head; "Модуль 8.
// Альтернативы Transformer", vladkulikov.com, section 7: with the transition
// a_t I the operator is the semi-separable matrix M_ij = C_i^T B_j
// prod_{r=j+1..i} a_r, which can be applied chunk by chunk with matrix
// products inside a chunk and the state passed between chunks; section 14:
// the state is [batch, nheads, headdim, d_state] and the input term dt B x):
//   for head h (group g = h / (nheads / ngroups)), channel p, step t:
//     dt = softplus(dt_in[b,t,h] + bias[h]);  a = exp(dt A[h])
//     s[p,n] <- a s[p,n] + dt B[b,t,g,n] x[b,t,h,p]
//     out[b,t,h,p] = (sum_n C[b,t,g,n] s[p,n] + D[h P + p] x) * silu(z)
//
// Chunked form used here, per (batch row, head) and chunk of Q = 32 steps with
// cumulative log-decay c_i = sum_{r<=i} dt_r A (log2 units, from the chunk start):
//   G    = C B^T                                  (Q x Q, over d_state)
//   W    = G o [j <= i] exp(c_i - c_j) dt_j         (causal decay mask)
//   Y    = diag(exp(c_i)) C S^T + W X             (S: state entering the chunk)
//   S^T <- exp(c_end) S^T + B^T (X o exp(c_end - c_j) dt_j)
// Every product runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  B,
// C and X are bf16 inputs, exact as operands.  W, the scaled X and the state
// are computed in fp32 and enter as two bf16 operands, hi = bf16(v) and
// lo = bf16(v - hi), whose products are summed: about 16 significant bits.
//
// Work decomposition (MI355X-first): a workgroup of four wavefronts owns one
// (batch row, head) and walks its chunks in order; wave w owns channels
// p in [16w, 16w + 16).  The state is held transposed, S^T [d_state x 16] per
// wave, in MFMA accumulators for the whole sequence.  Its accumulator layout
// (lane = channel, four consecutive n per lane and tile) is, up to a fixed
// permutation of n, the operand layout the readout C S^T needs; since that
// product sums over n, the C operand is read with the same permutation (two
// 8-byte LDS reads) and the state feeds the matrix cores straight from
// registers, never through LDS.  G is shared by the four waves (three 16 x 16
// tiles, one per wave) and reaches the W X product through LDS.  Every input
// is staged in LDS in its HBM layout (rows = steps) with 16-byte writes;
// operands whose contraction runs over time (B for the state update, x for
// both products) and the epilogue's x and z are read with gfx950's
// transposing LDS read, ds_read_b64_tr_b16: within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte pieces addressed by lanes
// 4e + i / 4 (e = 0..3), so lanes that address four rows of a row-major tile
// four columns apart receive its columns.  About 42 KiB of LDS per
// workgroup: three workgroups per CU.  The HBM reads of the next chunk are
// issued before the current chunk's arithmetic.
#include "device.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector (HIP's uint4 is a struct, whose copies the
// compiler routes through private memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kQ = 32;    // steps per chunk
constexpr int kP = 64;    // channels per head (headdim)

// Eight consecutive bf16 of a k-contiguous LDS row: one MFMA operand.
__device__ __forceinline__ bf16x8_t ld_op(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// Two runs of four bf16 (8 bytes each) joined into one operand.
__device__ __forceinline__ bf16x8_t ld_op2(const uint16_t* p0, const uint16_t* p1) {
  const bf16x4_t a = *reinterpret_cast<const bf16x4_t*>(p0);
  const bf16x4_t b = *reinterpret_cast<const bf16x4_t*>(p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposing read of 4 x 16-bit values (see the decomposition notes above).
__device__ __forceinline__ i16x4_t ld_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
}

// A column operand from a row-major tile: lane c of each 16-lane group gets
// rows r0 .. r0 + 7 of column c0 + c.  `tile` is the tile's first element,
// `stride` its row stride; lane l addresses row r0 + 4 half + (l % 16) / 4 and
// columns c0 + 4 (l % 4) .. + 3.
__device__ __forceinline__ bf16x8_t ld_col8(const uint16_t* tile, int stride, int r0, int c0, int l) {
  const int k = l & 15;
  const uint16_t* a0 = tile + (r0 + (k >> 2)) * stride + c0 + 4 * (k & 3);
  const i16x4_t lo = ld_tr(a0);
  const i16x4_t hi = ld_tr(a0 + 4 * stride);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two values as pairs of bf16 (hi = bf16(v), lo = bf16(v - hi)), packed with
// the first value in the low half: one conversion instruction per pair.
struct Split2 {
  uint32_t hi, lo;
};
__device__ __forceinline__ Split2 split_bf16x2(float v0, float v1) {
  const uint32_t hi = pack_bf16x2(v0, v1);
  return {hi, pack_bf16x2(v0 - __uint_as_float(hi << 16), v1 - __uint_as_float(hi & 0xffff0000u))};
}

// STATE_ONLY is pass A of a scan cut into time chunks: the chunk's end state
// from zero (chunk 0: from the initial state) and its summed log2 decay, with
// no readout and no output.  Otherwise time chunk blockIdx.z starts from the
// state the carry gives it (chunk 0: the initial state); with one chunk that
// is the whole sequence.
template <int N, typename Tout, bool STATE_ONLY>
__global__ void __launch_bounds__(256, 3) ssd_chunk_kernel(SsdArgs a) {
  constexpr int NT = N / 16;          // 16 x 16 state tiles per wave
  constexpr int NR = N / 64;          // 16-byte B/C vectors per thread and chunk
  constexpr int SC = N + 8;           // row strides (elements)
  constexpr int SB = N + 16;
  constexpr int SP = kP + 8;
  constexpr int SW = kQ + 8;
  __shared__ uint16_t sC[kQ * SC] __attribute__((aligned(16)));      // C[i][n]
  __shared__ uint16_t sB[kQ * SB] __attribute__((aligned(16)));      // B[j][n]
  __shared__ uint16_t sX[kQ * SP] __attribute__((aligned(16)));      // x[j][p]
  __shared__ uint16_t sZ[kQ * SP] __attribute__((aligned(16)));      // z[i][p]
  __shared__ uint16_t sXs[2][kQ * SP] __attribute__((aligned(16)));  // scaled x[j][p], hi/lo
  __shared__ uint16_t sW[2][kQ * SW] __attribute__((aligned(16)));   // W[i][j], hi/lo
  __shared__ float s_dt[kQ];                                          // step sizes dt_j
  __shared__ float s_cum[kQ];                                         // cumulative log2 decay c_j
  __shared__ float s_xs[kQ];                                          // exp(c_end - c_j) dt_j
  __shared__ float s_ec[kQ + 1];                                      // exp(c_i); [kQ]: exp(c_end)

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = l & 15, q = l >> 4;      // 16 x 16 tile: column / quarter of the lane
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int kt = blockIdx.z;                // time chunk
  const int K = a.n_chunks;
  const int H = a.nheads;
  const int G = a.ngroups;
  const int g = h / (H / G);
  const int64_t t_begin = (int64_t)kt * a.chunk_len;
  const int64_t L = min(a.chunk_len, a.seqlen - t_begin);   // steps of this time chunk
  const int64_t row0 = (int64_t)b * a.seqlen + t_begin;      // its first step, as a row of the batch
  const int64_t xrow = (int64_t)H * kP;     // elements between consecutive steps of x, z, out
  const int64_t bcrow = (int64_t)G * N;     // ... of B and C
  const uint16_t* xb = static_cast<const uint16_t*>(a.x) + row0 * xrow + (int64_t)h * kP;
  const uint16_t* zb = a.z ? static_cast<const uint16_t*>(a.z) + row0 * xrow + (int64_t)h * kP : nullptr;
  const uint16_t* dtb = static_cast<const uint16_t*>(a.dt) + row0 * H + h;
  const uint16_t* Bb = static_cast<const uint16_t*>(a.B) + row0 * bcrow + (int64_t)g * N;
  const uint16_t* Cb = static_cast<const uint16_t*>(a.C) + row0 * bcrow + (int64_t)g * N;
  Tout* ob = static_cast<Tout*>(a.out) + row0 * xrow + (int64_t)h * kP;
  const int64_t head_state = (int64_t)kP * N;   // state elements of one head
  const float A2 = a.A[h] * kLog2e;
  const float bias = a.bias ? a.bias[h] : 0.0f;
  const bool softplus = a.softplus != 0;
  const bool has_z = !STATE_ONLY && zb != nullptr;   // pass A reads neither z nor C
  const bool has_D = a.D != nullptr;
  const int p = 16 * w + lr;              // this lane's channel in the readout and the state
  const float Dp = has_D ? a.D[(int64_t)h * kP + p] : 0.0f;
  const uint32_t off_o = ((uint32_t)(4 * q) * (uint32_t)xrow + (uint32_t)p) * (uint32_t)sizeof(Tout);

  // Global loads and LDS staging: row-major 16-byte vectors (thread v covers
  // row v / (width / 8), vector v % (width / 8)); rows past the chunk's last
  // step re-read that step.  Addresses are a chunk base, uniform across the
  // workgroup and held in scalar registers, plus a per-lane 32-bit byte offset
  // that is the same for every full chunk: one chunk of any tensor spans less
  // than 2^31 bytes, since heads are at most 65535.
  const int xrow_i = tid >> 3, xc8 = tid & 7;
  const uint32_t bc_rowb = (uint32_t)bcrow * 2u, x_rowb = (uint32_t)xrow * 2u, dt_rowb = (uint32_t)H * 2u;
  auto bc_off = [&](int r, int nrow) SSM_INLINE {
    const int v = tid + 256 * r;
    return (uint32_t)min(v / (N / 8), nrow - 1) * bc_rowb + (uint32_t)(v % (N / 8)) * 16u;
  };
  uint32_t off_bc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) off_bc[r] = bc_off(r, kQ);
  const uint32_t off_x = (uint32_t)xrow_i * x_rowb + (uint32_t)xc8 * 16u;
  const uint32_t off_dt = (uint32_t)min(tid, kQ - 1) * dt_rowb;
  struct Bank {
    u32x4_t c[NR], bb[NR], x, z;
    uint32_t dt;
  };
  Bank bank;
  auto issue = [&](int64_t t0, int nt) SSM_INLINE {
    const char* Bc = reinterpret_cast<const char*>(Bb + t0 * bcrow);
    const char* Cc = reinterpret_cast<const char*>(Cb + t0 * bcrow);
    const char* xc = reinterpret_cast<const char*>(xb + t0 * xrow);
    const char* zc = has_z ? reinterpret_cast<const char*>(zb + t0 * xrow) : nullptr;
    const char* dtc = reinterpret_cast<const char*>(dtb + t0 * H);
    const bool full = nt == kQ;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t o = full ? off_bc[r] : bc_off(r, nt);
      if (!STATE_ONLY) bank.c[r] = *reinterpret_cast<const u32x4_t*>(Cc + o);
      bank.bb[r] = *reinterpret_cast<const u32x4_t*>(Bc + o);
    }
    const uint32_t ox = full ? off_x : (uint32_t)min(xrow_i, nt - 1) * x_rowb + (uint32_t)xc8 * 16u;
    bank.x = *reinterpret_cast<const u32x4_t*>(xc + ox);
    if (has_z) bank.z = *reinterpret_cast<const u32x4_t*>(zc + ox);
    if (tid < kQ)
      bank.dt = *reinterpret_cast<const uint16_t*>(dtc + (full ? off_dt : (uint32_t)min(tid, nt - 1) * dt_rowb));
  };

  // Stage the banked chunk (steps past nt carry x = 0 and dt = 0, so they
  // change nothing) and form the step sizes and per-step decay factors.
  float csum = 0.0f;   // wave 0: the summed log2 decay of the chunks so far
  auto stage = [&](int nt) SSM_INLINE {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int v = tid + 256 * r;
      const int row = v / (N / 8), c8 = v % (N / 8);
      if (!STATE_ONLY) *reinterpret_cast<u32x4_t*>(&sC[row * SC + c8 * 8]) = bank.c[r];
      *reinterpret_cast<u32x4_t*>(&sB[row * SB + c8 * 8]) = bank.bb[r];
    }
    if (xrow_i >= nt) bank.x = u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(&sX[xrow_i * SP + xc8 * 8]) = bank.x;
    if (has_z) *reinterpret_cast<u32x4_t*>(&sZ[xrow_i * SP + xc8 * 8]) = bank.z;
    if (w == 0) {
      float d = 0.0f;
      if (l < nt) {
        const float u = bf16_to_f32(bank.dt) + bias;
        d = softplus ? softplus_f(u) : u;
      }
      float one = 1.0f, c = d * A2;
      affine_wave_scan(one, c);  // (1, c) pairs compose to prefix sums of c
      // steps past nt add nothing, so the prefix at the last step is c_end
      const float c_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), kQ - 1));
      csum += c_end;
      if (l < kQ) {
        s_dt[l] = d;
        s_cum[l] = c;
        s_xs[l] = __builtin_amdgcn_exp2f(c_end - c) * d;
        s_ec[l] = __builtin_amdgcn_exp2f(c);
      }
      if (l == kQ) s_ec[kQ] = __builtin_amdgcn_exp2f(c_end);
    }
  };

  // The state S^T: tile t holds n in [16t, 16t + 16) x this wave's 16 channels;
  // register r of lane l is S^T[16t + 4(l/16) + r][p].
  const float* hsrc = kt == 0 ? (a.h0 != nullptr ? a.h0 + ((int64_t)b * H + h) * head_state : nullptr)
                     : STATE_ONLY ? nullptr
                     : a.ws_state + ((int64_t)(b * K + kt - 1) * H + h) * head_state;
  f32x4_t accS[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (hsrc != nullptr) {
      const float4 v = *reinterpret_cast<const float4*>(hsrc + (int64_t)p * N + 16 * t + 4 * q);
      accS[t] = f32x4_t{v.x, v.y, v.z, v.w};
    } else {
      accS[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  bool has_state = hsrc != nullptr;

  // W is zero above the diagonal: its block (rows 0..15, columns 16..31) is
  // never written by the chunks, so clear it once.
  for (int e = tid; e < 2 * 16 * 16; e += 256) {
    const int k = e >> 8, i = (e >> 4) & 15, j = 16 + (e & 15);
    sW[k][i * SW + j] = 0;
  }

  // D skip, gate and store of this lane's eight outputs (steps 16 ib + 4q + r
  // of channel p); the D and z switches are uniform and taken once per chunk,
  // and only a ragged last chunk checks its steps.
  auto finish = [&](const f32x4_t* accY, auto d_c, auto z_c, int nt, int64_t t0) SSM_INLINE {
    float y[2][4];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      // rows 16 ib + 4q .. + 3 of column p: one transposing read each
      const int k = l & 15;
      const int off = (16 * ib + 4 * q + (k >> 2)) * SP + 16 * w + 4 * (k & 3);
      i16x4_t xv = {0, 0, 0, 0}, zv = {0, 0, 0, 0};
      if (decltype(d_c)::value) xv = ld_tr(&sX[off]);
      if (decltype(z_c)::value) zv = ld_tr(&sZ[off]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = accY[ib][r];
        if (decltype(d_c)::value) v = __builtin_fmaf(Dp, bf16_to_f32((uint16_t)xv[r]), v);
        if (decltype(z_c)::value) v = v * silu_f(bf16_to_f32((uint16_t)zv[r]));
        y[ib][r] = v;
      }
    }
    // out: chunk base (scalar) + row base 16 ib + r (scalar) + this lane's 32-bit offset
    Tout* oc = ob + t0 * xrow;
    if (nt == kQ) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Io<Tout>::store(reinterpret_cast<char*>(oc + (16 * ib + r) * xrow) + off_o, 0, y[ib][r]);
    } else {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * ib + 4 * q + r < nt)
            Io<Tout>::store(reinterpret_cast<char*>(oc + (16 * ib + r) * xrow) + off_o, 0, y[ib][r]);
    }
  };

  const int64_t nchunks = (L + kQ - 1) / kQ;
  const ProgressPriority prio(nchunks);
  issue(0, (int)min((int64_t)kQ, L));
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    if (a.fair) prio.at(ch);
    const int64_t t0 = ch * kQ;
    const int nt = (int)min((int64_t)kQ, L - t0);
    stage(nt);
    const u32x4_t xreg = bank.x;        // this thread's staged x vector, for the scaled copy
    if (ch + 1 < nchunks) issue(t0 + kQ, (int)min((int64_t)kQ, L - t0 - kQ));
    block_sync();

    // Phase 1.  Waves 0..2: one 16 x 16 tile of G each, masked and decayed into W.
    if (!STATE_ONLY && w < 3) {
      const int ib = w == 0 ? 0 : 1, jb = w == 2 ? 1 : 0;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < N / 32; ++m)
        acc = mfma(ld_op(&sC[(16 * ib + lr) * SC + 32 * m + 8 * q]), ld_op(&sB[(16 * jb + lr) * SB + 32 * m + 8 * q]),
                   acc);
      const int j = 16 * jb + lr;
      const float cj = s_cum[j], dj = s_dt[j];
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * q + r;
        v[r] = j <= i ? acc[r] * __builtin_amdgcn_exp2f(s_cum[i] - cj) * dj : 0.0f;
      }
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const int i = 16 * ib + 4 * q + r;
        const Split2 sp = split_bf16x2(v[r], v[r + 1]);
        sW[0][i * SW + j] = (uint16_t)(sp.hi & 0xffffu);
        sW[0][(i + 1) * SW + j] = (uint16_t)(sp.hi >> 16);
        sW[1][i * SW + j] = (uint16_t)(sp.lo & 0xffffu);
        sW[1][(i + 1) * SW + j] = (uint16_t)(sp.lo >> 16);
      }
    }
    // The decayed, dt-weighted x of the state update, from this thread's own
    // staged vector: row j = xrow_i, channels 8 xc8 .. + 7, as hi/lo.
    {
      const float sc = s_xs[xrow_i];
      u32x4_t hv, lv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const Split2 sp = split_bf16x2(bf16_to_f32(xreg[e] & 0xffffu) * sc, __uint_as_float(xreg[e] & 0xffff0000u) * sc);
        hv[e] = sp.hi;
        lv[e] = sp.lo;
      }
      *reinterpret_cast<u32x4_t*>(&sXs[0][xrow_i * SP + xc8 * 8]) = hv;
      *reinterpret_cast<u32x4_t*>(&sXs[1][xrow_i * SP + xc8 * 8]) = lv;
    }
    // The readout of the incoming state, Y = diag(exp(c_i)) C S^T, from the
    // state registers: tiles 2m and 2m + 1 give the eight k slots of product m
    // (n = 32m + 4q + 0..3 and 32m + 16 + 4q + 0..3), and C is read with the
    // same n order.
    f32x4_t accY[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) accY[ib] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (!STATE_ONLY && has_state) {
#pragma unroll
      for (int m = 0; m < N / 32; ++m) {
        u32x4_t hw, lw;
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const Split2 s0 = split_bf16x2(accS[2 * m][r], accS[2 * m][r + 1]);
          const Split2 s1 = split_bf16x2(accS[2 * m + 1][r], accS[2 * m + 1][r + 1]);
          hw[r / 2] = s0.hi;
          lw[r / 2] = s0.lo;
          hw[2 + r / 2] = s1.hi;
          lw[2 + r / 2] = s1.lo;
        }
        const bf16x8_t shi = __builtin_bit_cast(bf16x8_t, hw);
        const bf16x8_t slo = __builtin_bit_cast(bf16x8_t, lw);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          const uint16_t* crow = &sC[(16 * ib + lr) * SC + 32 * m + 4 * q];
          const bf16x8_t ca = ld_op2(crow, crow + 16);
          accY[ib] = mfma(ca, shi, accY[ib]);
          accY[ib] = mfma(ca, slo, accY[ib]);
        }
      }
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) accY[ib][r] *= s_ec[16 * ib + 4 * q + r];
    }
    block_sync();

    // Phase 2.  Y += W X; D skip, gate and store; the state moves to the end
    // of the chunk.
    if constexpr (!STATE_ONLY) {
      const bf16x8_t xo = ld_col8(sX, SP, 8 * q, 16 * w, l);   // x[8q .. 8q + 7][p]
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        accY[ib] = mfma(ld_op(&sW[0][(16 * ib + lr) * SW + 8 * q]), xo, accY[ib]);
        accY[ib] = mfma(ld_op(&sW[1][(16 * ib + lr) * SW + 8 * q]), xo, accY[ib]);
      }
      if (has_D && has_z) finish(accY, std::true_type(), std::true_type(), nt, t0);
      else if (has_D) finish(accY, std::true_type(), std::false_type(), nt, t0);
      else if (has_z) finish(accY, std::false_type(), std::true_type(), nt, t0);
      else finish(accY, std::false_type(), std::false_type(), nt, t0);
    }
    {
      const float e_end = s_ec[kQ];
      const bf16x8_t xh = ld_col8(sXs[0], SP, 8 * q, 16 * w, l);   // scaled x[8q .. 8q + 7][p]
      const bf16x8_t xl = ld_col8(sXs[1], SP, 8 * q, 16 * w, l);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4_t acc = accS[t];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= e_end;
        const bf16x8_t bt = ld_col8(sB, SB, 8 * q, 16 * t, l);     // B[8q .. 8q + 7][16t + lr]
        acc = mfma(bt, xh, acc);
        acc = mfma(bt, xl, acc);
        accS[t] = acc;
      }
    }
    has_state = true;
    block_sync();
  }

  float* sdst = STATE_ONLY ? a.ws_state + ((int64_t)(b * K + kt) * H + h) * head_state
               : kt == K - 1 && a.state != nullptr ? a.state + ((int64_t)b * H + h) * head_state : nullptr;
  if (sdst != nullptr) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<float4*>(sdst + (int64_t)p * N + 16 * t + 4 * q) =
          make_float4(accS[t][0], accS[t][1], accS[t][2], accS[t][3]);
  }
  if (STATE_ONLY && tid == 0) a.ws_decay[(int64_t)(b * K + kt) * H + h] = csum;
}

// The carry of a scan cut into time chunks.  A head's decay over a chunk is
// the scalar exp2(summed log2 decay), so the pair (decay, end state) of every
// chunk composes in time order into the state entering the next chunk:
// S <- exp2(decay_k) S + end_k, from S = 0 (chunk 0's pair already carries the
// initial state).  One thread per (batch row, head, state element),
// sequential over chunks; slot k is replaced by the state entering chunk k + 1.
__global__ void __launch_bounds__(256) ssd_carry_kernel(SsdArgs a) {
  const int64_t per = (int64_t)a.headdim * a.d_state;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int h = (int)blockIdx.y;
  const int64_t b = blockIdx.z;
  if (e >= per) return;
  const int K = a.n_chunks, H = a.nheads;
  float S = 0.0f;
  for (int k = 0; k + 1 < K; ++k) {
    const int64_t slot = (b * K + k) * H + h;
    S = __builtin_fmaf(__builtin_amdgcn_exp2f(a.ws_decay[slot]), S, a.ws_state[slot * per + e]);
    a.ws_state[slot * per + e] = S;
  }
}

// ------------------------------------------------------------ decode step
//
// One step for every (b, h, p): the state row [N] is read and written once
// (16 bytes per lane, N / 4 lanes per row), the readout is reduced across
// those lanes with butterfly shuffles, and the row's first lane finishes y.
// Each thread takes two rows of one head, channels p and p + kSsdRowStride
// (kSsdRowStride = rows per 256 threads), which share the head's step, decay
// and B/C values: both rows' loads are issued before either row's arithmetic.
// (One row per thread took the batch-64 step of a 2.7B-like layer 69.6 us.)
template <typename Tin, typename Tout, int N>
__global__ void __launch_bounds__(256) ssd_update_kernel(SsdArgs a) {
  constexpr int LPR = N / 4;   // lanes per state row
  constexpr int RPB = 256 / LPR;  // rows per 256 threads: the stride between a thread's two rows
  // grid: x = blocks of 2 * RPB channels of one head, y = head, z = batch row
  // (the indices come from the grid, with no division by runtime sizes)
  const int p0 = (int)(blockIdx.x * (2 * RPB) + threadIdx.x / LPR);
  const int q = (int)(threadIdx.x % LPR);
  const int P = a.headdim, H = a.nheads, G = a.ngroups;
  if (p0 >= P) return;                    // whole rows leave together
  const int h = (int)blockIdx.y;
  const int64_t b = blockIdx.z;
  const int64_t bh = b * H + h;
  const int g = h / (H / G);              // uniform in the workgroup
  const int64_t bc = (b * G + g) * N + 4 * q;
  float Bv[4], Cv[4];
  load4<Tin>(a.B, bc, Bv);
  load4<Tin>(a.C, bc, Cv);
  // the second row may lie past the head (headdim not a multiple of 2 RPB):
  // it then re-reads the first row and stores nothing
  const bool live1 = p0 + RPB < P;
  int64_t row[2];
  row[0] = bh * P + p0;                   // (b * H + h) * P + p
  row[1] = live1 ? row[0] + RPB : row[0];
  float4 s4[2];
  float x[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    s4[r] = load_stream4(a.state + row[r] * N + 4 * q);  // the state streams, as in the Mamba-1 decode
    x[r] = ld_in(static_cast<const Tin*>(a.x) + row[r]);
  }
  const float u = ld_in(static_cast<const Tin*>(a.dt) + bh) + (a.bias ? a.bias[h] : 0.0f);
  const float dt = a.softplus ? softplus_f(u) : u;
  const float ar = __builtin_amdgcn_exp2f(dt * a.A[h] * kLog2e);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (r == 1 && !live1) break;
    const float dtx = dt * x[r];
    float hs[4] = {s4[r].x, s4[r].y, s4[r].z, s4[r].w};
    float y = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hs[i] = __builtin_fmaf(ar, hs[i], dtx * Bv[i]);
      y = __builtin_fmaf(Cv[i], hs[i], y);
    }
    store_stream4(a.state + row[r] * N + 4 * q, make_float4(hs[0], hs[1], hs[2], hs[3]));
    // The row's readout over its LPR lanes (16 or 32, aligned to the 16-lane
    // DPP rows): quad permutes, then the 8- and 16-lane mirrors leave each
    // 16-lane row's sum in all its lanes; with 32 lanes, row_bcast:15 adds the
    // first half's sum into the second, whose first lane then holds the total.
    y += SSM_DPP(0.0f, y, 0xB1, 0xf);   // quad_perm [1,0,3,2]
    y += SSM_DPP(0.0f, y, 0x4E, 0xf);   // quad_perm [2,3,0,1]
    y += SSM_DPP(0.0f, y, 0x141, 0xf);  // row_half_mirror
    y += SSM_DPP(0.0f, y, 0x140, 0xf);  // row_mirror
    if constexpr (LPR == 32) y += SSM_DPP(0.0f, y, 0x142, 0xa);  // row_bcast:15 into rows 1 and 3
    static_assert(LPR == 16 || LPR == 32, "the readout sum assumes 16 or 32 lanes per row");
    constexpr int kOut = LPR == 32 ? 16 : 0;  // the lane that holds the row's total
    if (q == kOut) {
      const int p = r == 0 ? p0 : p0 + RPB;
      if (a.D) y = __builtin_fmaf(a.D[(int64_t)h * P + p], x[r], y);
      if (a.z) y = y * silu_f(ld_in(static_cast<const Tin*>(a.z) + row[r]));
      Io<Tout>::store(a.out, row[r], y);
    }
  }
}

// One launch of a chunk-kernel instance, with the progress-priority scheme
// (ProgressPriority) on when the device holds the whole grid at once.
template <typename Kern>
void launch_ssd_pass(Kern kern, int per_cu, dim3 grid, const SsdArgs& a, hipStream_t s) {
  SsdArgs b = a;
  b.fair = grid_coresident(per_cu, a.cus, grid) ? 1 : 0;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, b);
}

template <int N, typename Tout>
void launch_ssd_nt(const SsdArgs& a, hipStream_t s) {
  static const int per_cu = resident_per_cu(ssd_chunk_kernel<N, Tout, false>, 256);
  static const int per_cu_a = resident_per_cu(ssd_chunk_kernel<N, float, true>, 256);
  if (a.n_chunks > 1) {
    launch_ssd_pass(ssd_chunk_kernel<N, float, true>, per_cu_a,
                    dim3((unsigned)a.nheads, (unsigned)a.batch, (unsigned)(a.n_chunks - 1)), a, s);
    const unsigned blocks = (unsigned)(((int64_t)a.headdim * a.d_state + 255) / 256);
    hipLaunchKernelGGL(ssd_carry_kernel, dim3(blocks, (unsigned)a.nheads, (unsigned)a.batch), dim3(256), 0, s, a);
  }
  launch_ssd_pass(ssd_chunk_kernel<N, Tout, false>, per_cu,
                  dim3((unsigned)a.nheads, (unsigned)a.batch, (unsigned)a.n_chunks), a, s);
}

template <int N>
void launch_ssd_n(const SsdArgs& a, DT out, hipStream_t s) {
  if (out == DT::F32) launch_ssd_nt<N, float>(a, s);
  else launch_ssd_nt<N, uint16_t>(a, s);
}

template <typename Tin, typename Tout>
void launch_ssd_update_t(const SsdArgs& a, hipStream_t s) {
  const int rows_per_block = 2 * (256 / (a.d_state / 4));  // two rows per thread
  const dim3 grid((unsigned)((a.headdim + rows_per_block - 1) / rows_per_block), (unsigned)a.nheads,
                  (unsigned)a.batch);
  if (a.d_state == 64) hipLaunchKernelGGL((ssd_update_kernel<Tin, Tout, 64>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ssd_update_kernel<Tin, Tout, 128>), grid, dim3(256), 0, s, a);
}

}  // namespace

hipError_t launch_ssd(const SsdArgs& a, DT out, hipStream_t s) {
  if (a.d_state == 64) launch_ssd_n<64>(a, out, s);
  else launch_ssd_n<128>(a, out, s);
  return hipGetLastError();
}

hipError_t launch_ssd_update(const SsdArgs& a, DT in, DT out, hipStream_t s) {
  if (in == DT::F32 && out == DT::F32) launch_ssd_update_t<float, float>(a, s);
  else if (in == DT::F32 && out == DT::BF16) launch_ssd_update_t<float, uint16_t>(a, s);
  else if (in == DT::BF16 && out == DT::F32) launch_ssd_update_t<uint16_t, float>(a, s);
  else launch_ssd_update_t<uint16_t, uint16_t>(a, s);
  return hipGetLastError();
}

}  // namespace ssm
