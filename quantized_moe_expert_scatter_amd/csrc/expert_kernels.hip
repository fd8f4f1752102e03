// expert_kernels.hip -- the two expert products (gate/up and down) for gfx950.
//
// "Strata" PR #3752 (commit list, Approach): one launch per product covers all
// experts; workgroups take row chunks of the experts from a chunk table,
// largest expert first, each expert at its own row count; each weight block is
// decoded once per pass; every product keeps the int8 values, the scales and
// a per-32-value fp32 epilogue in K order, the integer sum of a 32-value
// block being exact.  PR #2145 (description): Q2_0 weights, int32 sums exact
// in any order, a kernel bound by its fp32 epilogue rather than its matrix
// unit.
//
// gfx950 design (fp16 matrix cores, weights in registers, activations in LDS):
//  * A workgroup is one chunk of up to 128 expert-sorted activation rows of
//    one expert against 256 of that expert's weight rows (the N tile); each of
//    its 4 wavefronts owns 64 weight rows (two 32-row tiles).
//  * For each 64-value K stage the workgroup converts the chunk's q8_1 values
//    to fp16 once and stages them in LDS (double buffered; four lanes read
//    one row's 64 contiguous bytes, and one conversion per value picks and
//    packs the signed byte); each wavefront decodes its own weight blocks
//    straight into MFMA operand registers, so every weight block is decoded
//    exactly once and never round-trips through LDS, and every activation
//    operand read from LDS feeds both of the wave's weight tiles.
//  * Q2_0 decode: the tiled layout keeps, in each byte of a lane's code
//    word, two codes in the low bits of its nibbles (and two more above
//    them); after one mask a nibble 00cc read as FP4 (E2M1) is c/2, so one
//    FP4 -> fp16 conversion gives two values and one packed fp16 fma with
//    {2d, 2d} and {-2d, -2d} turns them into d*(c-2), exactly (two
//    instructions per two weights, a mask per eight).
//  * The contraction runs on v_mfma_f32_32x32x16_f16: a 32-value block is two
//    MFMAs (the second accumulating onto the first), 16 results per lane.
//    The activation q (int8) is exact in fp16; a Q2_0 weight d*(c-2) is exact
//    in fp16 (d is binary16, c-2 in {-2..1}).  Every partial sum of a
//    32-value block is an integer multiple of d's last bit below 2^24 in
//    magnitude, so the pair returns d*dot exactly -- the exact int32 block
//    dot scaled by the block's weight scale -- whatever order the matrix unit
//    adds in.  The per-32-value epilogue
//        acc = fmaf(dx, d * dot, acc)
//    is then one VALU operation per (row, output, block), bit for bit the
//    oracle's.  NL4 codebook entries are exact in fp16 too; there the MFMA
//    returns the dot itself and the epilogue is fmaf(dx, d * dot, acc) with
//    the product rounded once, as the oracle rounds it.
//    (The kernel is bound by VALU issue -- the epilogue FMAs, the weight
//    decode and the activation staging, four cycles per wave64 instruction --
//    with the MFMAs hidden under that stream only if they are spread out: an
//    MFMA issued while the previous one still runs stalls its wave, so two
//    issued back to back add about a fifth to a VALU-only stream at this
//    ratio of MFMA to VALU cycles, and the same MFMAs each followed by about
//    32 cycles of vector work add a twentieth (two waves per SIMD, measured).)
//  * MFMA operands: A = weights (lane l: weight row l%32), B = activations
//    (lane l: activation row l%32); lane half kq = l/32 holds values
//    16g + 8kq + p (p < 8) of a 32-value block in the MFMA of half g.  Any
//    assignment that A and B share gives the same exact sum; this one reads
//    the Q2_0 codes of block h from word h of the lane's bytes 8kq..8kq+7
//    (weight_pack.hip places them there), NL4 nibble g of the same bytes,
//    and 16 contiguous activation bytes.  A lane's 16 results share one
//    activation row (one dx per block) and cover weight rows
//    8q + 4kq + i (q, i < 4), stored as four float4.
//  * A chunk's last 32-row activation tile runs with the MFMA operands
//    swapped (activations as A), so its epilogue FMAs cover only the rows of
//    its 8-row steps; its results are transposed back through LDS at the end.
//  * Raw weight and activation bytes are loaded 2 stages ahead of their use
//    (5 for chunks of at most 64 rows, whose registers allow it); every load
//    is unconditional, so no in-flight register is copied (a copy would make
//    the compiler wait for every outstanding load).  Q2_0 loads go through
//    buffer descriptors (one per expert's weights, one per chunk's rows): a
//    lane's offset stays in a register, the stage's offset is a scalar, so
//    the loop computes no 64-bit addresses, and the descriptor's range check
//    keeps every access inside the expert or the chunk.  The descriptor's
//    base and range are read from the first lane, which tells the compiler
//    they are wave-uniform (without that it kept some descriptors in vector
//    registers and looped over their lanes for every load).  NL4 weights go
//    through the same descriptors.
//  * Work lists are grouped per XCD (workgroup id i runs on XCD i % 8): all
//    chunks of an expert land on one XCD, so its weight tiles and activation
//    rows are re-read from that XCD's L2.  Where every chunk has at most 64
//    rows, an item of the fp32-output products takes several N tiles of its
//    chunk as one stream of stages, so only its first tile waits for the
//    item's table reads and first weight loads.
#include "internal.h"
#include "q8_1.cuh"
#include "swiglu.cuh"

#include <hip/hip_runtime.h>

#include <type_traits>

namespace moe {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kKS = 64;                 // contraction values per stage
constexpr int kARow = kKS * 2 + 16;     // LDS bytes per staged activation row (padded)
constexpr int kMaxRows = 128;           // activation rows per chunk (4 tiles of 32)
constexpr int kWaves = 4;               // each owns 64 weight rows of the 256-row N tile

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ v2h as_v2h(uint32_t x) {
    v2h r;
    __builtin_memcpy(&r, &x, 4);
    return r;
}

__device__ __forceinline__ uint32_t as_u32(v2h x) {
    uint32_t r;
    __builtin_memcpy(&r, &x, 4);
    return r;
}

__device__ __forceinline__ v8h pack8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    v8h r;
    const uint32_t w[4] = {a, b, c, d};
    __builtin_memcpy(&r, w, 16);
    return r;
}

// 4 int8 -> 4 fp16 (two packed pairs), exact: byte b becomes the fp16
// 1024 + (b ^ 0x80) = 1152 + q, then 1152 is subtracted.
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, uint32_t &lo, uint32_t &hi) {
    const uint32_t u = w ^ 0x80808080u;
    const v2h bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    lo = as_u32(as_v2h(perm(0x64646464u, u, 0x05010400u)) + bias);
    hi = as_u32(as_v2h(perm(0x64646464u, u, 0x07030602u)) + bias);
}

// 4 int8 -> 4 fp16 (two packed pairs), exact, for the LDS staging: one
// conversion per value, the signed byte picked and packed by the instruction
// itself.  (Its results only go to LDS: the compiler does not see inside the
// asm, so it must not feed a matrix-core operand directly.)
__device__ __forceinline__ void i8x4_to_f16_staged(uint32_t w, uint32_t &lo, uint32_t &hi) {
    asm("v_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
        "v_cvt_f16_i16_sdwa %0, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
        "v_cvt_f16_i16_sdwa %1, sext(%2) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_f16_i16_sdwa %1, sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
        : "=&v"(lo), "=&v"(hi)
        : "v"(w));
}

// Q2_0 in the tiled layout: byte k of a lane's code word holds two codes in
// each nibble's low bits (bits 0-1 and 4-5) and two more above them (bits
// 2-3 and 6-7).  Masked to one pair per byte, a nibble 00cc read as FP4
// (E2M1) is exactly c/2, so one conversion gives two fp16 values c/2 and one
// packed fma with {2d, 2d} and {-2d, -2d} gives d*(c-2): the exact product
// c*d - 2d is a binary16 (|2d| <= 65504), so its single rounding is exact.
template <int K>
__device__ __forceinline__ v2h fp4_pair(uint32_t m) {
    return __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 1.0f, K));
}

// `word` is the lane's code word of 32-value block h; h[k] gets the fp16
// weights of values p = 2k, 2k + 1 of the lane's eight in MFMA g.
template <int G>
__device__ __forceinline__ void q2_decode8(uint32_t word, uint32_t d2, uint32_t nd2, uint32_t (&h)[4]) {
    const uint32_t m = (G == 0 ? word : word >> 2) & 0x33333333u;
    const v2h a = as_v2h(d2), c = as_v2h(nd2);
    h[0] = as_u32(__builtin_elementwise_fma(fp4_pair<0>(m), a, c));
    h[1] = as_u32(__builtin_elementwise_fma(fp4_pair<1>(m), a, c));
    h[2] = as_u32(__builtin_elementwise_fma(fp4_pair<2>(m), a, c));
    h[3] = as_u32(__builtin_elementwise_fma(fp4_pair<3>(m), a, c));
}

// NL4: four 4-bit codes (low nibbles of the bytes of c) -> four int8
// codebook entries: two byte-select lookups (entries 0-7 and 8-15) merged
// on bit 3 of each code (selector 0x0C yields 0x00, 0x0D yields 0xFF).
__device__ __forceinline__ uint32_t nl4_lookup(uint32_t c, const uint32_t (&cb)[4]) {
    const uint32_t lo3 = c & 0x07070707u;
    const uint32_t lo = perm(cb[1], cb[0], lo3);
    const uint32_t hi = perm(cb[3], cb[2], lo3);
    const uint32_t mask = perm(0u, 0u, ((c >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
    return (hi & mask) | (lo & ~mask);
}

__device__ __forceinline__ _Float16 half_bits(uint32_t h) {
    const uint16_t b = uint16_t(h);
    _Float16 v;
    __builtin_memcpy(&v, &b, 2);
    return v;
}

// Raw weight bytes of one lane for one stage and one 32-row weight tile:
// bytes 8kq..8kq+7 of the stage's block (Q2_0: one 64-value block, all four
// fields; NL4: the same bytes of each of the two 32-value blocks) and the
// scale(s) of the lane's weight row.
struct WRaw {
    uint2 c0, c1;
    uint32_t s;
};

// Raw bytes of one staged activation block: 32 q bytes and the scale.
struct ARaw {
    uint4 q0, q1;
    float d;
};

// The 8 fp16 weights lane half kq feeds to MFMA g of 32-value block h of the
// stage: values 16g + 8kq + p of the block.  Q2_0 (block h is half h of the
// 64-value block): field 2h + g of code bytes 8kq + p.  NL4 block h: nibble g
// of code bytes 8kq + p.
template <int WTYPE, int H, int G>
__device__ __forceinline__ v8h decode_ops(const WRaw &w, uint32_t thi, uint32_t tlo, const uint32_t (&cb)[4]) {
    uint32_t r[4];
    if constexpr (WTYPE == 1) {
        q2_decode8<G>(H == 0 ? w.c0.x : w.c0.y, thi, tlo, r);
    } else {
        const uint2 c = H == 0 ? w.c0 : w.c1;
        constexpr int sh = 4 * G;
        i8x4_to_f16(nl4_lookup((c.x >> sh) & 0x0F0F0F0Fu, cb), r[0], r[1]);
        i8x4_to_f16(nl4_lookup((c.y >> sh) & 0x0F0F0F0Fu, cb), r[2], r[3]);
    }
    return pack8(r[0], r[1], r[2], r[3]);
}

// The decode constants of a Q2_0 block scale d: thi = {2d, 2d} (exact: |2d|
// is at most 65504) and tlo = {-2d, -2d}.
__device__ __forceinline__ void q2_table(uint32_t hb, uint32_t &thi, uint32_t &tlo) {
    const uint32_t d = hb & 0xFFFFu;
    const v2h two = {(_Float16)2.0f, (_Float16)2.0f};
    thi = as_u32(as_v2h(d | (d << 16)) * two);
    tlo = thi ^ 0x80008000u;
}

// LDS offset of quarter i of a thread's staging: quarters 0-1 are its
// 16 values of row A, quarters 2-3 the same values of row B (64 rows on).
constexpr int stage_off(int i) { return i < 2 ? 16 * i : 64 * kARow + 16 * (i - 2); }

// Quarter i of the staging of one thread's activations: 8 q bytes to fp16 in LDS.
__device__ __forceinline__ void stage_piece(const ARaw &a, int i, uint8_t *dst) {
    const uint32_t q[8] = {a.q0.x, a.q0.y, a.q0.z, a.q0.w, a.q1.x, a.q1.y, a.q1.z, a.q1.w};
    uint4 o;
    i8x4_to_f16_staged(q[2 * i], o.x, o.y);
    i8x4_to_f16_staged(q[2 * i + 1], o.z, o.w);
    *reinterpret_cast<uint4 *>(dst + stage_off(i)) = o;
}

// Convert one thread's staged activations to fp16 and store them in LDS
// (NQ = 2: row A only, for chunks of at most 64 rows).
template <int NQ>
__device__ __forceinline__ void stage_acts(const ARaw &a, uint8_t *dst, float *dx) {
    const uint32_t q[8] = {a.q0.x, a.q0.y, a.q0.z, a.q0.w, a.q1.x, a.q1.y, a.q1.z, a.q1.w};
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        uint4 o;
        i8x4_to_f16_staged(q[2 * i], o.x, o.y);
        i8x4_to_f16_staged(q[2 * i + 1], o.z, o.w);
        *reinterpret_cast<uint4 *>(dst + stage_off(i)) = o;
    }
    *dx = a.d;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

constexpr int kTP = 36;                 // floats per row of the transposed tile (padded)

struct Lds {
    uint8_t act[2][kMaxRows * kARow];   // staged fp16 activations, double buffered
    float dx[2][2][kMaxRows];           // their block scales: [buffer][block of the stage][row]
    _Float16 dw[kWaves][2][2][32];      // NL4: block scales of each wave's weight rows
    float tp[kWaves][2][24][kTP];       // each wave's transposed last row tile (at most 24 rows)
};

// One stage (two 32-value blocks h) of Q2_0 outputs, software pipelined as
// one stream of MFMA pairs n = (h, r, t) (activation tile r, weight tile t).
// Pair n's two MFMAs are issued apart, each followed by half of the vector
// work that overlaps them: the epilogue of pair n-1 (eight FMAs after each
// MFMA; for the first pair, the previous stage's last pair, carried in
// prev / pdx), the next row tile's operands read from LDS as soon as their
// last reader has issued, a quarter of the next stage's activation staging,
// the decode of weight tile 1's block 0 (under the first pair) and of each
// tile's block 1 once its block 0 registers are dead, and the next stage's
// weight tables.  A matrix-core instruction issued while the previous one
// still runs stalls its wave until the unit is free; spaced by about 32
// cycles of vector work, each one issues at once and the two units stay busy
// together.  Scheduling barriers keep that order, with an empty volatile asm
// use of each MFMA result: the MFMA builtins are pure, and without it the
// compiler sank both MFMAs of a pair past the FMAs and barriers below them.
//
// QL < 4: the last row tile holds at most 8 QL of the chunk's rows and runs
// with the operands swapped (activations as A, weights as B; both use the
// same lane layout), so a lane's 16 results are its weight row against
// activation rows 8q + 4kq + i (q, i < 4) and only the 4 QL results of the
// rows q < QL get an epilogue FMA.  Those FMAs take one scale per row, read
// from LDS per block into dxv[h] (QL float4 per block); the item transposes
// the tile's accumulators back before its stores.
template <int NA, int QL>
__device__ __forceinline__ void stage_q2_pipelined(v16f (&acc)[2][NA], const WRaw (&w)[2], const WRaw (&wn)[2],
                                                   uint32_t (&thi)[2], uint32_t (&tlo)[2], const ARaw &anext,
                                                   uint8_t *sdst, float *sdx, const uint8_t *arow0,
                                                   const float *dxrow0, const float *dxt0, v16f &prev, float &pdx,
                                                   v4f (&dxv)[2][4]) {
    constexpr int NP = 4 * NA;                    // pairs in the stage
    constexpr bool TR = QL < 4;                   // row tile NA-1 runs transposed
    const uint32_t cb[4] = {0u, 0u, 0u, 0u};
    // the scales of the transposed tile's rows for block h
    auto read_dxv = [&](int h) {
#pragma unroll
        for (int q = 0; q < QL; ++q) dxv[h][q] = *reinterpret_cast<const v4f *>(dxt0 + h * kMaxRows + 8 * q);
    };
    // operands of the first row tile of block 0 and tile 0's block-0 weights;
    // tile 1's are decoded under the first pair
    v8h b0 = *reinterpret_cast<const v8h *>(arow0);
    v8h b1 = *reinterpret_cast<const v8h *>(arow0 + 32);
    float dx = 0.0f;
    if constexpr (TR && NA == 1)
        read_dxv(0);
    else
        dx = dxrow0[0];
    v8h wop[2][2];
    wop[0][0] = decode_ops<1, 0, 0>(w[0], thi[0], tlo[0], cb);
    wop[0][1] = decode_ops<1, 0, 1>(w[0], thi[0], tlo[0], cb);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NP>([&](auto NN) {
        constexpr int n = decltype(NN)::value;
        constexpr int h = n / (2 * NA), r = (n >> 1) % NA, t = n & 1;
        constexpr bool tr = TR && r == NA - 1;
        // pair n-1 (for n = 0 the previous stage's last pair, carried in)
        constexpr int pr = n > 0 ? ((n - 1) >> 1) % NA : NA - 1, pt = n > 0 ? (n - 1) & 1 : 1;
        constexpr int ph = n > 0 ? (n - 1) / (2 * NA) : 1;
        constexpr bool ptr = TR && pr == NA - 1;
        // the operands that follow this row tile: (h, r+1) or (1, 0)
        constexpr bool next = t == 1 && (r + 1 < NA || h == 0);
        constexpr int nh = r + 1 < NA ? h : 1, nr = r + 1 < NA ? r + 1 : 0;
        constexpr bool ntr = TR && nr == NA - 1;
        const uint8_t *nsrc = arow0 + nr * 32 * kARow + 64 * nh;
        // block 1's weights of tile dt: half 0 right after the last pair of
        // tile dt in block 0, half 1 one pair later
        constexpr int dec0 = n >= 2 * NA - 2 && n < 2 * NA ? n - (2 * NA - 2) : -1;
        constexpr int dec1 = n >= 2 * NA - 1 && n < 2 * NA + 1 ? n - (2 * NA - 1) : -1;
        // epilogue FMAs of pair n-1 in each half
        constexpr int F = ptr ? 2 * QL : 8;

        // first half: MFMA 0 of the pair, then the reads of the next row
        // tile's first operand and scale, staging or a table, the first
        // half of pair n-1's FMAs
        v16f p = tr ? __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, wop[t][0], v16f{}, 0, 0, 0)
                    : __builtin_amdgcn_mfma_f32_32x32x16_f16(wop[t][0], b0, v16f{}, 0, 0, 0);
        asm volatile("" ::"v"(p));
        __builtin_amdgcn_sched_barrier(0);
        const float cdx = dx;
        if constexpr (next) {
            b0 = *reinterpret_cast<const v8h *>(nsrc);
            if constexpr (ntr)
                read_dxv(nh);
            else
                dx = dxrow0[nh * kMaxRows + nr * 32];
        }
        if constexpr (dec1 >= 0) wop[dec1][1] = decode_ops<1, 1, 1>(w[dec1], thi[dec1], tlo[dec1], cb);
        if constexpr (n == 0) wop[1][0] = decode_ops<1, 0, 0>(w[1], thi[1], tlo[1], cb);
        // a chunk of at most 64 rows stages row A only (quarters 0-1)
        constexpr int NQ = NA > 2 ? 4 : 2;
        static_for<0, NQ>([&](auto II) {
            constexpr int i = decltype(II)::value;
            constexpr int at = i * (4 / NQ) * NA + 1 < NP - 1 ? i * (4 / NQ) * NA + 1 : NP - 1;
            if constexpr (at == n) {
                stage_piece(anext, i, sdst);
                if constexpr (i == NQ - 1) *sdx = anext.d;
            }
        });
        // the next stage's table of tile t, once block 1 of tile t is decoded
        if constexpr (h == 1 && r == 0) q2_table(wn[t].s, thi[t], tlo[t]);
#pragma unroll
        for (int i = 0; i < F; ++i)
            acc[pt][pr][i] = __builtin_fmaf(ptr ? dxv[ph][i >> 2][i & 3] : pdx, prev[i], acc[pt][pr][i]);
        __builtin_amdgcn_sched_group_barrier(0x100, next ? (ntr ? 1 + QL : 2) : 0, 0);
        __builtin_amdgcn_sched_barrier(0);

        // second half: MFMA 1 (onto MFMA 0), the next second operand, the
        // rest of pair n-1's FMAs
        p = tr ? __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, wop[t][1], p, 0, 0, 0)
               : __builtin_amdgcn_mfma_f32_32x32x16_f16(wop[t][1], b1, p, 0, 0, 0);
        asm volatile("" ::"v"(p));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (next) b1 = *reinterpret_cast<const v8h *>(nsrc + 32);
        if constexpr (dec0 >= 0) wop[dec0][0] = decode_ops<1, 1, 0>(w[dec0], thi[dec0], tlo[dec0], cb);
        if constexpr (n == 0) wop[1][1] = decode_ops<1, 0, 1>(w[1], thi[1], tlo[1], cb);
#pragma unroll
        for (int i = F; i < 2 * F; ++i)
            acc[pt][pr][i] = __builtin_fmaf(ptr ? dxv[ph][i >> 2][i & 3] : pdx, prev[i], acc[pt][pr][i]);
        __builtin_amdgcn_sched_group_barrier(0x100, next ? 1 : 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        prev = p;
        pdx = cdx;
    });
    // the stage's last pair is left in prev / pdx (dxv[1] when transposed)
    // for the next stage's first unit (or the item's end)
}

constexpr int kOut = 0;     // fp32 outputs
constexpr int kDots = 1;    // the int32 block dots (test export)
constexpr int kSwiglu = 2;  // gate/up with swiglu and q8_1 of H in the epilogue

// Four rounded values t[0..3] (binary32 whose truncation toward zero is the
// q value, in [-127, 127]) converted and packed, value k in byte k.
__device__ __forceinline__ uint32_t pack_trunc_i8x4(float t0, float t1, float t2, float t3) {
    const uint32_t lo = perm(uint32_t(int32_t(t1)), uint32_t(int32_t(t0)), 0x0C0C0400u);
    const uint32_t hi = perm(uint32_t(int32_t(t3)), uint32_t(int32_t(t2)), 0x04000C0Cu);
    return lo | hi;
}

// q8_1 of one lane's 16 values of a 32-value block whose other 16 sit in
// lane ^ 32: d = max|x| / 127 (the fp32 divide), q = x / d rounded half away
// from zero and clamped to [-127, 127].  x / d is the correctly rounded
// binary32 quotient without a divide per value: r = 1/d in binary64 (one
// divide per block), then x * r rounded to binary64 and that to binary32.
// That is exact because the quotient of two binary32 values is never a
// binary32 rounding boundary and lies at least 2^-49 of its size away from
// one, while x * r is within 2^-52 of it.  The rounding adds +-0.49999997
// (the binary32 below 1/2) in binary32 and truncates: for every binary32 y
// in [-127, 127] that is y rounded half away from zero (checked for all of
// them), where adding 1/2 itself would round 0.49999997 up to 1.  q bytes
// are packed four to a word, value i of the lane in byte i % 4 of word
// i / 4, and s is summed from the packed bytes.
__device__ __forceinline__ void q8_1_half_block(const float (&x)[16], uint32_t (&w)[4], float &d,
                                                int32_t &sum) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
    d = amax / 127.0f;
    sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = 0u;
    if (d != 0.0f) {
        const double r = 1.0 / static_cast<double>(d);
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float y = static_cast<float>(static_cast<double>(x[i]) * r);
            const float yc = __builtin_amdgcn_fmed3f(y, -127.0f, 127.0f);
            t[i] = yc + __builtin_copysignf(0x1.fffffep-2f, yc);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w[k] = pack_trunc_i8x4(t[4 * k], t[4 * k + 1], t[4 * k + 2], t[4 * k + 3]);
            sum = __builtin_amdgcn_sdot4(int(w[k]), 0x01010101, sum, false);
        }
    }
    sum += __shfl_xor(sum, 32);
}

// Fused epilogue for one activation row: the lane holds gate (tile 0) and up
// (tile 1) of the same 16 j's, h = silu(g) * u exactly as swiglu_q8 computes
// it, and the 32-value q8_1 block of h is shared with lane ^ 32.
__device__ __forceinline__ void swiglu_store_row(const v16f &g, const v16f &u, uint8_t *hrow, int n_ff,
                                                 int jbase, int kq) {
    float h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        h[i] = silu_div(static_cast<double>(g[i]), 1.0f + exp_neg_rn32(g[i])) * u[i];
    }
    uint32_t w[4];
    float d;
    int32_t sum;
    q8_1_half_block(h, w, d, sum);
    // value i of the lane is j = jbase + 8 (i / 4) + 4 kq + i % 4
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t *>(hrow + jbase + 8 * q + 4 * kq) = w[q];
    if (kq == 0) {
        const int blk = jbase >> 5;
        reinterpret_cast<float *>(hrow + n_ff)[blk] = d;
        reinterpret_cast<int32_t *>(hrow + n_ff + 4 * (n_ff >> 5))[blk] = sum;
    }
}

// A pointer that is the same in every lane, read from the first lane so the
// compiler keeps it (and what is built from it) in scalar registers.
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return reinterpret_cast<const uint8_t *>((uint64_t(hi) << 32) | lo);
}

// The whole K loop of one work item.  Each wave owns 64 weight rows (two
// 32-row tiles) and runs them against NA 32-row activation tiles (the chunk's
// rows rounded up; rows past the chunk are never stored).  In the fused
// swiglu mode the item's tile is 128 j's: the wave's tile 0 is gate rows
// j0..j0+31 and its tile 1 the up rows n_ff+j0..n_ff+j0+31 of the same j's.
// QL < 4 (pipelined Q2_0 only): the last row tile holds at most 8 QL rows and
// runs transposed (see stage_q2_pipelined).
template <int WTYPE, int MODE, int NA, int QL>
__device__ __forceinline__ void run_item(const ProductArgs &a, Lds &L, int expert, int row0,
                                         int nrows, int n0, int nt) {
    constexpr bool DOTS = MODE == kDots;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int kq = lane >> 5;                    // k half of the MFMA operands
    const int col = lane & 31;
    const int cols = a.cols;
    const int nb32 = cols >> 5;
    const uint32_t arb = uint32_t(cols) + uint32_t(nb32) * 8u;
    constexpr int WB = WTYPE == 1 ? 64 : 32;
    const int nbw = cols / WB;
    const int n_stages = (cols + kKS - 1) / kKS;

    // weights (tiled layout: block b of row 32i + r at slot (i * nbw + b) * 32 + r):
    // this lane's row in each of the wave's two tiles (clamped for loads)
    const uint8_t *wexp = a.w_base + a.w_off[expert];
    const int n_ff = a.out_rows >> 1;
    const int nw = MODE == kSwiglu ? n0 + 32 * wave : n0 + 64 * wave;
    // weight rows (j's in the fused mode) from one N tile to the next
    constexpr int tstep = MODE == kSwiglu ? kTileRows / 2 : kTileRows;
    const int wlimit = MODE == kSwiglu ? n_ff : a.out_rows;
    bool wave_on = nw < wlimit;
    // first weight row of each of the wave's two tiles
    const int tb[2] = {nw, MODE == kSwiglu ? n_ff + nw : nw + 32};
    uint32_t coff[2], soff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t wr = uint32_t(min(tb[t] + col, a.out_rows - 1));
        soff[t] = (wr & ~31u) * uint32_t(nbw) + (wr & 31u);      // slot of block 0
        coff[t] = soff[t] * 16u + 8u * uint32_t(kq);
    }
    uint32_t cb[4] = {0u, 0u, 0u, 0u};
    if constexpr (WTYPE == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            cb[i] = uint32_t(uint8_t(a.codebook[4 * i])) | (uint32_t(uint8_t(a.codebook[4 * i + 1])) << 8) |
                    (uint32_t(uint8_t(a.codebook[4 * i + 2])) << 16) |
                    (uint32_t(uint8_t(a.codebook[4 * i + 3])) << 24);
    }
    // Items read the expert's two planes (codes, then scales) through one
    // buffer descriptor: the lane's offsets stay in registers, the stage's
    // offset is a scalar, and the descriptor's range keeps every access
    // inside the expert.  Q2_0: one 64-value block per stage; NL4: two
    // 32-value blocks (the second one 32 slots on, absent past the end of a
    // row of odd block count: its bytes are loaded but never used).
    const uint32_t codes_bytes = uint32_t(a.out_rows) * uint32_t(nbw) * 16u;
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void *)uniform_ptr(wexp), 0, __builtin_amdgcn_readfirstlane(int(codes_bytes + codes_bytes / 8u)),
        0x00020000);
    // An item's N tiles are whole tiles of the expert when it has more than
    // one: tile lt of the item is tile 0's rows moved by lt * tstep, which in
    // the tiled layout is a uniform byte shift of each plane.
    const int cshift = tstep * nbw * 16, sshift = tstep * nbw * 2;
    auto wload = [&](int stage, int t, int lt = 0) {
        const int s = min(stage, n_stages - 1);
        const int blk = s * (kKS / WB);                      // first block of the stage
        WRaw w;
        w.c0 = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(wres, coff[t], blk * 512 + lt * cshift, 0));
        if constexpr (WTYPE == 1) {
            w.c1 = w.c0;
            w.s = __builtin_amdgcn_raw_buffer_load_b16(wres, 2u * soff[t],
                                                       int(codes_bytes) + blk * 64 + lt * sshift, 0);
        } else {
            const int b1 = min(blk + 1, nbw - 1);            // the next block of the same 32 rows
            w.c1 = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(wres, coff[t], b1 * 512 + lt * cshift, 0));
            w.s = uint32_t(__builtin_amdgcn_raw_buffer_load_b16(wres, 2u * soff[t],
                                                                int(codes_bytes) + blk * 64 + lt * sshift, 0)) |
                  (uint32_t(__builtin_amdgcn_raw_buffer_load_b16(wres, 2u * soff[t],
                                                                 int(codes_bytes) + b1 * 64 + lt * sshift, 0))
                   << 16);
        }
        return w;
    };

    // rows 64-127 are staged only for chunks of more than 64 rows
    constexpr int NQ = NA > 2 ? 4 : 2;
    // activations: thread tid stages values 16p..16p+15 (p = tid&3) of the
    // stage in rows tid/4 and 64 + tid/4, so four lanes read one row's 64
    // contiguous bytes; it loads the scale of block p&1 of row tid/4 (p < 2)
    // or of row 64 + tid/4.  Rows past the chunk are not clamped: the
    // descriptor's range check returns zeros for them, so the padded rows of
    // the last tile are staged as zeros (the matrix core then multiplies
    // zeros, which costs less power than copies of a real row, and no load
    // goes to memory for them; their results are never stored).
    const int srow = tid >> 2;
    const int spc = tid & 3;
    const int drow = srow + 64 * (spc >> 1), dblk = spc & 1;
    const uint8_t *abase = a.act + size_t(row0) * arb;
    const uint32_t aoffA = uint32_t(srow) * arb;
    const uint32_t aoffB = uint32_t(srow + 64) * arb;
    const uint32_t aoffD = uint32_t(drow) * arb;
    // the chunk's rows through one descriptor (past the chunk the range
    // check returns zeros; the block after the last of a row of odd block
    // count reads the row's own scales and sums, staged but never used)
    const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
        (void *)uniform_ptr(abase), 0, __builtin_amdgcn_readfirstlane(int(uint32_t(nrows) * arb)), 0x00020000);
    const uint32_t aqA = aoffA + 16u * uint32_t(spc), aqB = aoffB + 16u * uint32_t(spc);
    const uint32_t ad = aoffD + uint32_t(cols) + 4u * uint32_t(dblk);
    auto aload = [&](int stage) {
        const int s = min(stage, n_stages - 1);
        ARaw r;
        r.q0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, aqA, 64 * s, 0));
        if constexpr (NQ == 4)
            r.q1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, aqB, 64 * s, 0));
        else
            r.q1 = uint4{0u, 0u, 0u, 0u};
        r.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ares, ad, 8 * s, 0));
        return r;
    };

    v16f acc[2][NA];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < NA; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][r][i] = 0.0f;

    // U register slots; the stage loop is unrolled by U so every slot is a
    // fixed register set.  The weights of stage x sit in wslot[x % U] and are
    // loaded U stages before use; the activations of stage x sit in
    // aslot[x % U], loaded U-1 stages before they are staged into LDS.  Each
    // stage issues its activation load before its weight load (vmcnt retires
    // loads in order).  Loads and staging run in every unrolled stage, past
    // the end too (clamped, never used), so that every path through the loop
    // has the same loads in flight and the compiler's waits stay exact; only
    // the compute is skipped.  Fewer activation tiles leave registers for a
    // deeper prefetch.
    constexpr bool PIPE = WTYPE == 1 && !DOTS;
    // (NL4 with four row tiles: one stage ahead; two would spill)
    constexpr int U = (WTYPE == 2 && NA == 4) ? 1 : (NA >= 3 ? 2 : kStreamU);
    // the pipelined stage computes the next stage's weight tables from the
    // next slot, which must then hold the next stage (not this one)
    static_assert(!PIPE || U >= 2, "pipelined Q2_0 stages need two or more prefetch slots");
    WRaw wslot[U][2];
    ARaw aslot[U];
    // the prologue issues the slots' loads in the loop's own order (the
    // scheduler would otherwise group them by base address): the waits at the
    // loop head merge this path with the back edge, so any load that trails
    // here shortens the prefetch of every iteration
#pragma unroll
    for (int x = 0; x < U; ++x) {
        aslot[x] = aload(x);
#pragma unroll
        for (int t = 0; t < 2; ++t) wslot[x][t] = wload(x, t);
        __builtin_amdgcn_sched_barrier(0);
    }
    stage_acts<NQ>(aslot[0], &L.act[0][srow * kARow + 32 * spc], &L.dx[0][dblk][drow]);
    // the pipelined Q2_0 stage computes the next stage's weight tables itself
    uint32_t pthi[2] = {0u, 0u}, ptlo[2] = {0u, 0u};
    if constexpr (PIPE) {
#pragma unroll
        for (int t = 0; t < 2; ++t) q2_table(wslot[0][t].s, pthi[t], ptlo[t]);
    }
    __syncthreads();

    // the pipelined stage's last MFMA pair, whose epilogue runs under the
    // next stage's first pair (zero before the first stage: fmaf(0, 0, +0)
    // leaves the accumulator +0)
    v16f cprev;
#pragma unroll
    for (int i = 0; i < 16; ++i) cprev[i] = 0.0f;
    float cpdx = 0.0f;
    // the transposed tile's row scales per block (QL < 4); zero like cpdx,
    // since the first stage's carried FMAs read dxv[1]
    v4f dxv[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) dxv[h][q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Stage s of the current tile, its LDS buffer par (the parity of the
    // stage's index in the item's stream); slot j takes the loads of stage ls
    // of the item's tile lt, U stages on.
    auto stage = [&](auto J, int s, int par, int ls, int lt) {
        constexpr int j = decltype(J)::value;
        constexpr int jn = (j + 1) % U;
        const int k0 = s * kKS;
        const int nv = min(kKS, cols - k0);
        const int nblk = WTYPE == 1 ? 2 : (nv >> 5);
        // slot j's activations were staged at the end of the previous stage
        // (or before the loop), so it takes the load U stages on now
        aslot[j] = aload(ls);

        if constexpr (PIPE) {
            if (wave_on && s < n_stages)
                stage_q2_pipelined<NA, QL>(acc, wslot[j], wslot[jn], pthi, ptlo, aslot[jn],
                                           &L.act[par ^ 1][srow * kARow + 32 * spc], &L.dx[par ^ 1][dblk][drow],
                                           L.act[par] + col * kARow + 16 * kq, &L.dx[par][0][col],
                                           &L.dx[par][0][32 * (NA - 1) + 4 * kq], cprev, cpdx, dxv);
            else
                stage_acts<NQ>(aslot[jn], &L.act[par ^ 1][srow * kARow + 32 * spc], &L.dx[par ^ 1][dblk][drow]);
#pragma unroll
            for (int t = 0; t < 2; ++t) wslot[j][t] = wload(ls, t, lt);
            __syncthreads();
            return;
        }
        if (wave_on && s < n_stages) {
            uint32_t thi[2] = {0u, 0u}, tlo[2] = {0u, 0u};
            if constexpr (WTYPE == 1) {
#pragma unroll
                for (int t = 0; t < 2; ++t) q2_table(DOTS ? 0x3C00u : wslot[j][t].s, thi[t], tlo[t]);
            } else {
                // publish this lane's row scales for the epilogue
                if (kq == 0) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        L.dw[wave][0][t][col] = half_bits(wslot[j][t].s & 0xFFFFu);
                        L.dw[wave][1][t][col] = half_bits(wslot[j][t].s >> 16);
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
            const uint8_t *abuf = L.act[par];
            static_for<0, 2>([&](auto HH) {
                constexpr int h = decltype(HH)::value;
                if (h < nblk) {
                    v8h wop[2][2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        wop[t][0] = decode_ops<WTYPE, h, 0>(wslot[j][t], thi[t], tlo[t], cb);
                        wop[t][1] = decode_ops<WTYPE, h, 1>(wslot[j][t], thi[t], tlo[t], cb);
                    }
                    // NL4: the lane's 16 weight-row scales of each tile, binary16
                    v4h dwv[2][4];
                    if constexpr (WTYPE == 2) {
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                dwv[t][q] = *reinterpret_cast<const v4h *>(&L.dw[wave][h][t][8 * q + 4 * kq]);
                    }
#pragma unroll
                    for (int r = 0; r < NA; ++r) {
                        const uint8_t *src = abuf + (r * 32 + col) * kARow + (32 * h + 8 * kq) * 2;
                        const v8h b0 = *reinterpret_cast<const v8h *>(src);
                        const v8h b1 = *reinterpret_cast<const v8h *>(src + 32);
                        const float dx = L.dx[par][h][r * 32 + col];
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            v16f p = __builtin_amdgcn_mfma_f32_32x32x16_f16(wop[t][0], b0, v16f{}, 0, 0, 0);
                            p = __builtin_amdgcn_mfma_f32_32x32x16_f16(wop[t][1], b1, p, 0, 0, 0);
                            if constexpr (DOTS) {
                                const int arow = r * 32 + col;
                                const int rr = row0 + arow - a.dots_row_begin;
                                if (arow < nrows && rr >= 0 && rr < a.dots_n_rows) {
#pragma unroll
                                    for (int i = 0; i < 16; ++i) {
                                        const int wrow = nw + 32 * t + 8 * (i >> 2) + 4 * kq + (i & 3);
                                        a.dots[(size_t(rr) * a.out_rows + wrow) * nb32 + (k0 >> 5) + h] = int(p[i]);
                                    }
                                }
                            } else if constexpr (WTYPE == 1) {
#pragma unroll
                                for (int i = 0; i < 16; ++i) acc[t][r][i] = __builtin_fmaf(dx, p[i], acc[t][r][i]);
                            } else {
                                // dw * dot rounded once (an fma onto -0 is the plain
                                // product, signed zeros included), then the epilogue fma
#pragma unroll
                                for (int i = 0; i < 16; ++i) {
                                    const float wd = __builtin_fmaf(static_cast<float>(dwv[t][i >> 2][i & 3]), p[i], -0.0f);
                                    acc[t][r][i] = __builtin_fmaf(dx, wd, acc[t][r][i]);
                                }
                            }
                        }
                    }
                }
            });
        }

        stage_acts<NQ>(aslot[jn], &L.act[par ^ 1][srow * kARow + 32 * spc], &L.dx[par ^ 1][dblk][drow]);
#pragma unroll
        for (int t = 0; t < 2; ++t) wslot[j][t] = wload(ls, t, lt);
        __syncthreads();
    };

    // The item's nt N tiles of the chunk as one stream of stages: the groups
    // of U stages line up with the tiles (the launch takes nt > 1 only where U
    // divides the stage count), and the last group of a tile issues the loads
    // of the next tile's first U stages, so that tile starts with its data in
    // flight; each tile ends with its epilogue and clears its accumulators.
    // (only items of at most 64 rows with fp32 outputs stream: in larger
    // items the prefetch slots would stay live through every tile's epilogue,
    // beside the larger accumulators, and spill; the fused mode's items are
    // long enough without)
    constexpr bool STREAM = PIPE && MODE == kOut && NA <= 2;
    const int ntt = STREAM ? nt : 1;
    int gpar = 0;                                        // parity of the stream's stage index
    for (int ti = 0; ti < ntt; ++ti) {
        const int nwt = nw + ti * tstep;                 // this wave's first weight row (j) in tile ti
        wave_on = nwt < wlimit;
        for (int s0 = 0; s0 < n_stages; s0 += U) {
            const bool nx = s0 + U >= n_stages && ti + 1 < ntt;
            const int lb = nx ? s0 + U - n_stages : s0 + U;
            const int lt = nx ? ti + 1 : ti;
            static_for<0, U>([&](auto J) {
                constexpr int jj = decltype(J)::value;
                stage(J, s0 + jj, (gpar + jj) & 1, lb + jj, lt);
            });
            gpar = (gpar + U) & 1;
        }

        if constexpr (PIPE) {
            if (wave_on) {
                if constexpr (QL < 4) {
#pragma unroll
                    for (int i = 0; i < 4 * QL; ++i)
                        acc[1][NA - 1][i] = __builtin_fmaf(dxv[1][i >> 2][i & 3], cprev[i], acc[1][NA - 1][i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[1][NA - 1][i] = __builtin_fmaf(cpdx, cprev[i], acc[1][NA - 1][i]);
                }
            }
        }
        if constexpr (QL < 4) {
            // The transposed tile back to the MFMA layout the stores take,
            // through the wave's own LDS area: lane l holds weight row l%32
            // against activation rows 8q + 4kq + i, and reads back activation
            // row l%32 (clamped: rows past 8 QL are past the chunk, never
            // stored) against weight rows 8q + 4kq + i.
            if (wave_on) {
                float(&tp)[2][24][kTP] = L.tp[wave];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4 * QL; ++i)
                        tp[t][8 * (i >> 2) + 4 * kq + (i & 3)][col] = acc[t][NA - 1][i];
                __builtin_amdgcn_wave_barrier();
                const int ar = min(col, 8 * QL - 1);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4f v = *reinterpret_cast<const v4f *>(&tp[t][ar][8 * q + 4 * kq]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[t][NA - 1][4 * q + i] = v[i];
                    }
                // the next tile's transpose writes this area again
                __builtin_amdgcn_wave_barrier();
            }
        }

        if constexpr (MODE == kSwiglu) {
            if (wave_on) {
                const size_t hrb = size_t(n_ff) + size_t(n_ff >> 5) * 8;
#pragma unroll
                for (int r = 0; r < NA; ++r) {
                    // lanes l and l ^ 32 hold the two halves of a block and share
                    // the activation row, so they skip rows past the chunk together
                    const int arow = r * 32 + col;
                    if (arow < nrows)
                        swiglu_store_row(acc[0][r], acc[1][r], a.hq + size_t(row0 + arow) * hrb, n_ff, nwt, kq);
                }
            }
        } else if constexpr (!DOTS) {
            if (wave_on) {
                // Stores of 16 rows x 64 contiguous bytes.  In the MFMA layout
                // lane l holds row l%32 of a tile and 4-float pieces 8q + 4kq of
                // it, so a store would cover 32 rows with 32 bytes each: into
                // rows scattered by the permutation, a pattern that the memory
                // system takes at half the rate of 64-byte pieces (measured
                // alone).  One 16-lane row swap between the registers of pieces
                // q = 2p and 2p + 1 (lanes 16-31 and 48-63 of the first with
                // lanes 0-15 and 32-47 of the second) leaves rows 0-15 of the
                // tile in the first register and rows 16-31 in the second, each
                // lane with the piece 16p + 4 (l / 32) + 8 ((l / 16) % 2) of row
                // l % 16 (+16).  The swaps run with every lane active; only the
                // stores are masked by the chunk's row count.
                const int sub = lane & 15;
                const int cpos = nwt + 4 * (lane >> 5) + 8 * ((lane >> 4) & 1);
#pragma unroll
                for (int r = 0; r < NA; ++r) {
                    v4f sw[2][2][2];                     // [t][pair p][rows 0-15, rows 16-31]
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int p = 0; p < 2; ++p)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float lo = acc[t][r][8 * p + i], hi = acc[t][r][8 * p + 4 + i];
                                const auto x = __builtin_amdgcn_permlane16_swap(
                                    __builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi), false,
                                    false);
                                sw[t][p][0][i] = __builtin_bit_cast(float, uint32_t(x[0]));
                                sw[t][p][1][i] = __builtin_bit_cast(float, uint32_t(x[1]));
                            }
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int arow = r * 32 + 16 * hf + sub;
                        if (arow < nrows) {
                            const int rr = row0 + arow;
                            const size_t orow = a.perm ? size_t(a.perm[rr]) : size_t(rr);
                            float *dst = a.out + orow * a.out_rows + cpos;
#pragma unroll
                            for (int t = 0; t < 2; ++t)
#pragma unroll
                                for (int p = 0; p < 2; ++p)
                                    *reinterpret_cast<v4f *>(dst + 32 * t + 16 * p) = sw[t][p][hf];
                        }
                    }
                }
            }
        }

        if (ti + 1 < ntt) {
            // the next tile starts from zero, and so does its first carried pair
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < NA; ++r)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[t][r][i] = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) cprev[i] = 0.0f;
            cpdx = 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int q = 0; q < 4; ++q) dxv[h][q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
}

// The pipelined Q2_0 items take the rows of their last 32-row tile in steps
// of 8 (1..4); the others always run whole tiles.
template <int WTYPE, int MODE, int NA>
__device__ __forceinline__ void run_item_rows(const ProductArgs &a, Lds &L, int expert, int row0, int nrows,
                                              int n0, int nt) {
    if constexpr (WTYPE == 1 && MODE != kDots) {
        const int last = nrows - 32 * (NA - 1);
        if (last <= 8)
            run_item<WTYPE, MODE, NA, 1>(a, L, expert, row0, nrows, n0, nt);
        else if (last <= 16)
            run_item<WTYPE, MODE, NA, 2>(a, L, expert, row0, nrows, n0, nt);
        else if (last <= 24)
            run_item<WTYPE, MODE, NA, 3>(a, L, expert, row0, nrows, n0, nt);
        else
            run_item<WTYPE, MODE, NA, 4>(a, L, expert, row0, nrows, n0, nt);
    } else {
        run_item<WTYPE, MODE, NA, 4>(a, L, expert, row0, nrows, n0, nt);
    }
}

template <int WTYPE, int MODE>
__global__ __launch_bounds__(256, 2) void expert_product_kernel(ProductArgs a) {
    __shared__ __attribute__((aligned(16))) Lds L;

    // work item: a chunk from this XCD's list and a group of a.group
    // consecutive weight tiles of it (the last group of a chunk may be short)
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds;
    const int j = bid / kXcds;
    const int xcnt = a.xcd[kXcds + xcd];
    const int grp = a.group > 1 ? a.group : 1;
    const int per_chunk = (a.n_tiles + grp - 1) / grp;
    if (j >= xcnt * per_chunk) return;
    const int c = a.xcd[xcd] + j / per_chunk;
    const int tile = (j % per_chunk) * grp;
    const int nt = min(grp, a.n_tiles - tile);
    const int expert = a.chunks[4 * c + 0];
    const int row0 = a.chunks[4 * c + 1];
    const int nrows = a.chunks[4 * c + 2];
    const int n0 = tile * (MODE == kSwiglu ? kTileRows / 2 : kTileRows);

    const int na = (nrows + 31) >> 5;          // 32-row activation tiles: 1..4
    if (na <= 1) {
        run_item_rows<WTYPE, MODE, 1>(a, L, expert, row0, nrows, n0, nt);
    } else if (na == 2) {
        run_item_rows<WTYPE, MODE, 2>(a, L, expert, row0, nrows, n0, nt);
    } else if (na == 3) {
        run_item_rows<WTYPE, MODE, 3>(a, L, expert, row0, nrows, n0, 1);
    } else {
        run_item_rows<WTYPE, MODE, 4>(a, L, expert, row0, nrows, n0, 1);
    }
}

hipError_t launch_expert_product(const ProductArgs &a, hipStream_t stream) {
    if (a.max_items <= 0) return hipSuccess;
    const dim3 grid(kXcds * a.max_items), block(64 * kWaves);
    if (a.wtype == 1) {
        if (a.dots)
            hipLaunchKernelGGL((expert_product_kernel<1, kDots>), grid, block, 0, stream, a);
        else if (a.hq)
            hipLaunchKernelGGL((expert_product_kernel<1, kSwiglu>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((expert_product_kernel<1, kOut>), grid, block, 0, stream, a);
    } else {
        if (a.dots)
            hipLaunchKernelGGL((expert_product_kernel<2, kDots>), grid, block, 0, stream, a);
        else if (a.hq)
            hipLaunchKernelGGL((expert_product_kernel<2, kSwiglu>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((expert_product_kernel<2, kOut>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace moe
