/*
 * cpattn -- per-rank attention for context-parallel diffusion transformers
 * on AMD Instinct MI355X (gfx950).  C ABI, version 4 (CPATTN_ABI_VERSION).
 *
 * What the library computes (sources are the pages' titles and sections):
 *
 *  - attn_fwd: non-causal multi-head scaled dot-product attention returning
 *    O and the per-row natural log-sum-exp of the scaled scores.  Diffusion
 *    transformers attend bidirectionally, with no causal mask ("Scaling AI
 *    inference across multiple GPUs using NVIDIA TensorRT with multi-device
 *    inference support", section "Context parallelism"); the score chain is
 *    scaled QK^T -> softmax -> times V with a total scale of 1/sqrt(head_dim)
 *    ("TensorRT multi-device attention inference in practice", step 1).
 *    Context parallelism divides this work per rank: AllGather-KV gives a
 *    rank its query rows against all keys, Ulysses gives it all rows of a
 *    head subset, and Ring Attention gives it one K/V chunk at a time (first
 *    page, sections "AllGather KV", "Ring Attention", "DeepSpeed Ulysses").
 *
 *  - attn_merge: combines two partial results (O, LSE) over disjoint key
 *    sets into the result over their union -- the online-softmax step that
 *    lets Ring Attention stream K/V chunks (first page, "Ring Attention").
 *
 *  - attn_fwd_ex: attn_fwd with a caller workspace (key-range split of the
 *    last, partial wave of query tiles, folded back with the same merge) and
 *    an accumulate mode that folds the result into an existing (O, LSE) --
 *    one Ring Attention step with the merge done in the attention epilogue.
 *
 *  - ring_attn_fwd: the per-rank ring loop on one device: attention of the
 *    local queries against each of n K/V chunks in turn, each chunk folded
 *    into the running (O, LSE) by the attn_merge rule (first page, "Ring
 *    Attention").
 *
 *  - attn_fwd_fp8: the same attention with 8-bit float (E4M3) inputs on the
 *    fp8 matrix cores.
 *
 *  - qk_rmsnorm: the QK-RMSNorm prologue (fp32 RMSNorm over head_dim, cast
 *    to the 16-bit type, split score scale) of the attention sample in
 *    "TensorRT multi-device attention inference in practice", step 1.
 *
 *  - ulysses_pack / ulysses_unpack (and the batched _n forms): the
 *    sequence<->head relayout on either side of DeepSpeed Ulysses' two
 *    all-to-alls (first page, "DeepSpeed Ulysses"; 5520 tokens per rank at
 *    degree 8 in "Simplifying model
 *    serving across multiple GPUs with NVIDIA TensorRT multi-device
 *    integration in NVIDIA Dynamo-Triton", section on distributing Cosmos 3
 *    with Ulysses context parallelism).
 *
 * Conventions shared by every entry point:
 *
 *  - Every tensor pointer is DEVICE memory owned by the caller, contiguous
 *    (row-major, last dimension fastest) and 16-byte aligned.  A call's
 *    buffers and stream belong to one device, which must be the calling
 *    thread's current HIP device (the per-device state below is kept for the
 *    current device).  The library
 *    never allocates, frees or retains caller memory and has no handles;
 *    scratch memory, where a call can use it, is a caller-owned workspace
 *    argument, except for cpattn_attn_fwd_ex_static, which uses a fixed
 *    device array of the library's own.  The other state kept between calls
 *    is a per-device cache of the number of attention workgroups the device
 *    holds at once and of that array's device address.
 *  - Work is enqueued on the caller's HIP stream (0 = the null stream) and
 *    runs asynchronously; the call returns once the launches are enqueued.
 *    A call enqueues kernels only (no memset, copy, allocation or
 *    synchronisation), so calls can be recorded into a HIP graph by stream
 *    capture; make one call on the device before capturing, so that the
 *    one-time per-device lookups described below run outside the capture.
 *  - Argument checks run synchronously, on the host, before any HIP call.
 *    A failed check returns its status and enqueues nothing.  A launch
 *    failure returns CPATTN_E_HIP.  Faults inside a kernel surface at the
 *    caller's next synchronisation on the stream.
 *  - Sizes are int64_t; every element count must stay below 2^62 and every
 *    per-dimension size below 2^31.
 *  - Functions are reentrant and thread-safe.  Calls on different streams
 *    may run concurrently as long as their buffers do not overlap (for
 *    cpattn_attn_fwd_ex_static that includes the library's scratch: see there).
 *
 * bf16 is the 16-bit brain-float format stored as raw 16-bit words; f16 is
 * IEEE binary16; f32 is IEEE binary32.
 */
#ifndef CPATTN_H_
#define CPATTN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPATTN_ABI_VERSION 4

/* Bytes of work counters at the head of an attention workspace. */
#define CPATTN_WORKSPACE_COUNTER_BYTES 2048

typedef enum {
    CPATTN_OK = 0,
    CPATTN_E_NULL = 1,     /* a required pointer is NULL                          */
    CPATTN_E_SHAPE = 2,    /* a size is out of range, inconsistent or overflows   */
    CPATTN_E_DTYPE = 3,    /* unsupported dtype or dtype combination              */
    CPATTN_E_HEADDIM = 4,  /* head dimension D not supported by the kernel        */
    CPATTN_E_ALIGN = 5,    /* a pointer is not 16-byte aligned                    */
    CPATTN_E_ALIAS = 6,    /* buffers overlap where overlap is not allowed        */
    CPATTN_E_HIP = 7,      /* the HIP runtime rejected a launch                   */
    CPATTN_E_SCALE = 8,    /* the score scale is not a finite positive number     */
    CPATTN_E_FLAGS = 9     /* unknown bits in a flags argument                    */
} cpattn_status;

/* Flags of cpattn_attn_fwd_ex. */
#define CPATTN_FLAG_ACCUMULATE 1u
#define CPATTN_FLAG_SEQ_MAJOR 2u
#define CPATTN_FLAG_K_SEQ_LAST 4u

/* CPATTN_E4M3 (OCP FP8 E4M3 bytes) is only an in_dtype of cpattn_attn_fwd_workspace_size:
 * cpattn_attn_fwd_fp8 takes no dtype for its inputs. */
typedef enum { CPATTN_BF16 = 0, CPATTN_F32 = 1, CPATTN_F16 = 2, CPATTN_E4M3 = 3 } cpattn_dtype;

typedef enum { CPATTN_SEQ_TO_HEAD = 0, CPATTN_HEAD_TO_SEQ = 1 } cpattn_dir;

/*
 * Non-causal attention forward with per-row LSE.
 *
 *   q   [B, H, Sq,  D]  in_dtype         k, v [B, H, Skv, D]  in_dtype
 *   o   [B, H, Sq,  D]  o_dtype (output)  lse  [B, H, Sq]      f32 (output)
 *
 *   z_ij   = scale * sum_d q_id k_jd
 *   LSE_i  = ln sum_j exp(z_ij)                 (computed max-shifted)
 *   O_id   = sum_j exp(z_ij - LSE_i) v_jd
 *
 * No mask of any kind.  Skv = 0 is allowed and yields O = 0, LSE = -inf
 * (the identity of attn_merge).  B, H, Sq >= 1; Skv >= 0; D in {64, 128};
 * scale finite and > 0 (1/sqrt(D) is the usual choice).
 *
 * dtypes: in_dtype = BF16 with o_dtype = BF16 (bf16 matrix cores, fp32
 * accumulation and softmax state, softmax weights rounded to bf16 for the PV
 * product, O rounded to nearest even) or o_dtype = F32 (the same computation
 * with O kept in f32, e.g. for ring partials); in_dtype = F16 with o_dtype =
 * F16 or F32, the same with IEEE fp16 in place of bf16 (the precision of the
 * attention sample in "TensorRT multi-device attention inference in
 * practice"); in_dtype = F32 requires o_dtype = F32 (all arithmetic in f32).
 * Any other pair -> CPATTN_E_DTYPE.
 *
 * o and lse must not overlap each other or q, k, v (CPATTN_E_ALIAS).
 */
cpattn_status cpattn_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                              float scale, cpattn_dtype in_dtype, cpattn_dtype o_dtype,
                              hipStream_t stream);

/*
 * attn_fwd with a caller workspace and flags.
 *
 * Same tensors, dtypes, results and checks as cpattn_attn_fwd, plus:
 *
 *   workspace        device memory, 16-byte aligned, workspace_bytes long, or
 *                    NULL with workspace_bytes = 0.  Contents on entry are
 *                    ignored and undefined on return.  Must not overlap any
 *                    tensor argument (CPATTN_E_ALIAS); NULL with a nonzero
 *                    size is CPATTN_E_NULL.
 *   flags            any of CPATTN_FLAG_ACCUMULATE, CPATTN_FLAG_SEQ_MAJOR,
 *                    CPATTN_FLAG_K_SEQ_LAST (not together with SEQ_MAJOR);
 *                    other bits or that pair -> CPATTN_E_FLAGS.
 *
 * Workspace.  The bf16 kernel runs 256 query rows of one (b, h) per
 * workgroup, at most one workgroup per resident slot, each looping over
 * units of work.  The first CPATTN_WORKSPACE_COUNTER_BYTES bytes of a
 * workspace hold work counters: after the first round, units are claimed
 * from them, each XCD from its own contiguous range of units first (its
 * workgroups then share each head's K and V in its L2), then from a tail
 * shared by all, so the XCDs that run faster (their clocks differ under the
 * power limit) take more of it (the call clears the counters itself, with a
 * kernel).
 * When the tiles do not fill the device's last wave, the keys of the tiles
 * in that wave are also split into pieces that run in parallel, and a
 * second kernel folds the pieces with the attn_merge rule.  The split is
 * planned per call from the device's resident-workgroup count and limited
 * to what the rest of the workspace holds: (D + 1) * 1024 bytes per piece.
 * cpattn_attn_fwd_workspace_size gives the size the best plan uses
 * (CPATTN_WORKSPACE_COUNTER_BYTES when no split helps); less only means
 * fewer (or no) pieces, and under CPATTN_WORKSPACE_COUNTER_BYTES (or none)
 * also the static unit order of cpattn_attn_fwd.
 * f32 inputs never split; bf16 and fp16 inputs share the plan.
 * Results differ from cpattn_attn_fwd's only by f32 rounding in the fold:
 * without a split the two give the same bits.
 *
 * CPATTN_FLAG_ACCUMULATE.  (o, lse) hold on entry the result of attention
 * over a disjoint key set (O normalised, f32; LSE natural; LSE = -inf with
 * O = 0 for "nothing yet"), and on return the result over the union:
 * each row is folded with the attn_merge rule in f32.  Requires in_dtype =
 * BF16 or F16 and o_dtype = F32 (else CPATTN_E_DTYPE).  With Skv = 0 the
 * call leaves (o, lse) unchanged.
 *
 * CPATTN_FLAG_SEQ_MAJOR.  q, k, v and o are sequence-major (token-major):
 * q [B, Sq, H, D], k and v [B, Skv, H, D], o [B, Sq, H, D]; lse stays
 * [B, H, Sq].  This is the layout of a rank's token shard and, with
 * H = H_total / P, of the DeepSpeed Ulysses receive buffer [P, S_local, H, D]
 * read as [S, H, D] (first page, "DeepSpeed Ulysses"): attention reads that
 * buffer in place and writes o straight into the send buffer of the second
 * all-to-all, so no relayout pass is needed on the head side.  Same results
 * as the head-major call on the transposed tensors, bit for bit.  A token
 * row (H * D elements) must be shorter than 2^25 elements (CPATTN_E_SHAPE).
 *
 * CPATTN_FLAG_K_SEQ_LAST.  k is [B, H, D, Skv]: each head's keys stored with
 * the sequence last, the layout the attention sample's sharding hint gives
 * K (K of rank 4 with its sequence at dimension 3, "TensorRT multi-device
 * attention inference in practice", the hint-file section); q, v and o stay
 * head-major [B, H, S, D].  The same arithmetic on the same tiles as with
 * k [B, H, Skv, D], so the same results, bit for bit.  Requires BF16 or F16
 * inputs (CPATTN_E_DTYPE), Skv a multiple of 8 and D * Skv * 2 < 2^32
 * (CPATTN_E_SHAPE).
 */
cpattn_status cpattn_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                 float scale, cpattn_dtype in_dtype, cpattn_dtype o_dtype,
                                 uint32_t flags, void* workspace, uint64_t workspace_bytes,
                                 hipStream_t stream);

/*
 * cpattn_attn_fwd_ex for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation: the split workspace is the library's static scratch instead
 * of a caller buffer, and the call allocates nothing.
 *
 * The scratch is a file-scope device array of CPATTN_STATIC_SCRATCH_BYTES
 * (32 MiB), one per device, held from the first call on that device until
 * the process ends; the first call on a device looks up its address there
 * (CPATTN_E_HIP if HIP cannot give it).  scratch_bytes is how much of it the
 * split may use, exactly as workspace_bytes for cpattn_attn_fwd_ex (0 = no
 * split; cpattn_attn_fwd_workspace_size gives the best plan's size, and a
 * smaller size only means fewer pieces); scratch_bytes above
 * CPATTN_STATIC_SCRATCH_BYTES -> CPATTN_E_SHAPE.  Every other argument,
 * check and result is that of cpattn_attn_fwd_ex: with the same
 * scratch_bytes as workspace_bytes the outputs are the same bits.
 *
 * Nothing in the scratch needs clearing by the caller: the call clears the
 * work counter at its head with a kernel of its own (no memset), and writes
 * every byte its piece merge reads before reading it, in stream order.  All calls
 * on one device share that device's scratch, so calls on one device must not
 * overlap in time (issue them on one stream, or order the streams): two
 * overlapping calls race on it.
 */
#define CPATTN_STATIC_SCRATCH_BYTES (32u << 20)

cpattn_status cpattn_attn_fwd_ex_static(const void* q, const void* k, const void* v, void* o, float* lse,
                                        int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                        float scale, cpattn_dtype in_dtype, cpattn_dtype o_dtype,
                                        uint32_t flags, uint64_t scratch_bytes, hipStream_t stream);

/*
 * Attention with 8-bit float inputs (OCP FP8 E4M3), one f32 scale per tensor.
 *
 *   q [B, H, Sq, D], k and v [B, H, Skv, D]  E4M3 bytes (real value = decoded byte * scale)
 *   o [B, H, Sq, D]  o_dtype = BF16 or F32 (else CPATTN_E_DTYPE)   lse [B, H, Sq] f32
 *   (with CPATTN_FLAG_SEQ_MAJOR: q, o [B, Sq, H, D], k, v [B, Skv, H, D]; lse unchanged)
 *
 * The result is attention (as cpattn_attn_fwd defines it, with `scale` on the scores) of
 * the real-valued tensors q * q_scale, k * k_scale, v * v_scale.  The pages name
 * quantisation as an inference optimisation ("Scaling AI inference across multiple GPUs
 * using NVIDIA TensorRT with multi-device inference support", opening section) but give
 * no recipe; this one runs both products on gfx950's fp8 matrix cores (twice the bf16
 * rate) with f32 scores and softmax state, and rounds the softmax weights to E4M3 (as
 * p * 2^7, p <= 2) for the PV product.  D = 128 only (CPATTN_E_HEADDIM); scales finite
 * and > 0 (CPATTN_E_SCALE); flags: any of CPATTN_FLAG_SEQ_MAJOR and
 * CPATTN_FLAG_ACCUMULATE (else CPATTN_E_FLAGS; sequence-major needs H * D < 2^25,
 * else CPATTN_E_SHAPE; accumulate, as for cpattn_attn_fwd_ex, needs o_dtype = F32,
 * else CPATTN_E_DTYPE).  workspace / workspace_bytes as for cpattn_attn_fwd_ex (work
 * counter, then key-range pieces); cpattn_attn_fwd_workspace_size with in_dtype =
 * CPATTN_E4M3 gives the best plan's size.  Skv = 0 gives O = 0, LSE = -inf (or leaves
 * an accumulated result unchanged).  Other checks as for cpattn_attn_fwd.
 */
cpattn_status cpattn_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, float scale,
                                  float q_scale, float k_scale, float v_scale, cpattn_dtype o_dtype,
                                  uint32_t flags, void* workspace, uint64_t workspace_bytes,
                                  hipStream_t stream);

/*
 * Workspace bytes cpattn_attn_fwd_ex (in_dtype BF16 or F16) or cpattn_attn_fwd_fp8
 * (in_dtype E4M3, o_dtype BF16 or F32, D = 128) uses for this problem on the CURRENT
 * device (CPATTN_WORKSPACE_COUNTER_BYTES for the work counters when no split helps;
 * 0 for f32 inputs).  Makes HIP queries of
 * the current device (CU count, kernel occupancy); CPATTN_E_HIP if they fail.
 * Shape checks as for cpattn_attn_fwd (the scale is not needed).
 */
cpattn_status cpattn_attn_fwd_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                             cpattn_dtype in_dtype, cpattn_dtype o_dtype,
                                             uint64_t* bytes);

/*
 * The split plan of cpattn_attn_fwd_ex (bf16 inputs) for a device that holds
 * `slots` attention workgroups at once, with workspace_bytes of workspace.
 * Host only, no HIP call.  Outputs: split_tiles = number of trailing query
 * tiles split (0 = no split), pieces = pieces per split tile (1 if none),
 * bytes_used = workspace the plan uses (the 256-byte work counter plus the
 * pieces; 0 when workspace_bytes < 256).  slots = 0 means "unknown" (no
 * split).  Shape checks as for cpattn_attn_fwd.
 */
cpattn_status cpattn_attn_fwd_split_plan(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                         int64_t slots, uint64_t workspace_bytes,
                                         int64_t* split_tiles, int64_t* pieces, uint64_t* bytes_used);

/*
 * Merge two partial attention results over disjoint key sets a and b.
 *
 *   o_a, o_b, o_out  [B, H, S, D]  o_dtype      lse_a, lse_b, lse_out  [B, H, S]  f32
 *
 *   M   = max(La, Lb)
 *   L   = M + ln(exp(La - M) + exp(Lb - M))
 *   O   = exp(La - L) * Oa + exp(Lb - L) * Ob
 *
 * computed in f32 and stored in o_dtype (BF16, F16 or F32; 16-bit types
 * rounded to nearest even).
 * An empty side (LSE = -inf, O = 0) is the identity; two empty sides give
 * O = 0, LSE = -inf.  o_out may be exactly o_a or exactly o_b, and lse_out
 * exactly lse_a or lse_b (in-place accumulation); any other overlap is
 * CPATTN_E_ALIAS.  B, H, S >= 1; D >= 8 with D*sizeof(o_dtype) a multiple of
 * 16 bytes and D <= 1024.
 */
cpattn_status cpattn_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                                void* o_out, float* lse_out, int64_t B, int64_t H, int64_t S, int64_t D,
                                cpattn_dtype o_dtype, hipStream_t stream);

/*
 * Ring Attention on one rank, stream-ordered on one device.
 *
 *   q         [B, H, Sq, D]                      bf16
 *   k_chunks  [n_chunks, B, H, Skv_chunk, D]     bf16  (chunk c = the c-th block of keys
 *   v_chunks  [n_chunks, B, H, Skv_chunk, D]     bf16   a ring would deliver)
 *   o         [B, H, Sq, D]  f32 (output)          lse  [B, H, Sq] f32 (output)
 *   o_work    [B, H, Sq, D]  f32 (caller-owned scratch, or NULL)
 *   lse_work  [B, H, Sq]     f32 (caller-owned scratch, or NULL; NULL exactly
 *                                 when o_work is NULL, else CPATTN_E_NULL)
 *
 * Chunk 0's attention is written to (o, lse); every later chunk's attention
 * is folded into (o, lse) in its epilogue with the attn_merge rule (f32), as
 * cpattn_attn_fwd_ex with CPATTN_FLAG_ACCUMULATE does.  The work buffers, when
 * given, serve as the workspace (the work counters in the first
 * CPATTN_WORKSPACE_COUNTER_BYTES bytes of lse_work, which must be at least
 * that long to be used; the key-range pieces in the rest; contents undefined
 * on return).  The result equals attention over the concatenation of all
 * chunks.  n_chunks >= 1, Skv_chunk >= 0, D in {64, 128}, scale as for
 * attn_fwd.  o, lse, o_work and lse_work must not overlap each other or the
 * inputs.
 */
cpattn_status cpattn_ring_attn_fwd(const void* q, const void* k_chunks, const void* v_chunks,
                                   float* o, float* lse, float* o_work, float* lse_work,
                                   int64_t B, int64_t H, int64_t Sq, int64_t Skv_chunk, int64_t n_chunks,
                                   int64_t D, float scale, hipStream_t stream);

/*
 * Ulysses relayout, packing side (builds the all-to-all send buffer).
 * Hp = H / P, S = P * S_local.
 *
 *   SEQ_TO_HEAD: src [B, S_local, H, D]  ->  dst [B, P, S_local, Hp, D]
 *                dst[b,p,s,h,:] = src[b,s,p*Hp+h,:]
 *   HEAD_TO_SEQ: src [B, Hp, S, D]       ->  dst [B, P, S_local, Hp, D]
 *                dst[b,p,s,h,:] = src[b,h,p*S_local+s,:]
 *
 * Chunk p of dst is destined for rank p.  A bit-exact copy of elements of
 * type dt.  H % P == 0 (else CPATTN_E_SHAPE); D*sizeof(dt) a multiple of 16
 * bytes (else CPATTN_E_HEADDIM) and below 2^35 bytes, B*S_local*H at most
 * 2^32 - 1 rows (else CPATTN_E_SHAPE); src and dst must not overlap.  Rank r
 * is taken to own tokens
 * [r*S_local, (r+1)*S_local) and heads [r*Hp, (r+1)*Hp).
 */
cpattn_status cpattn_ulysses_pack(const void* src, void* dst, int64_t B, int64_t S_local, int64_t H,
                                  int64_t D, int64_t P, cpattn_dtype dt, cpattn_dir dir,
                                  hipStream_t stream);

/*
 * Ulysses relayout, unpacking side (reads the all-to-all receive buffer,
 * whose chunk p came from rank p).
 *
 *   SEQ_TO_HEAD: src [B, P, S_local, Hp, D]  ->  dst [B, Hp, S, D]
 *                dst[b,h,p*S_local+s,:] = src[b,p,s,h,:]
 *   HEAD_TO_SEQ: src [B, P, S_local, Hp, D]  ->  dst [B, S_local, H, D]
 *                dst[b,s,g*Hp+h,:] = src[b,g,s,h,:]
 *
 * Same requirements as cpattn_ulysses_pack.
 */
cpattn_status cpattn_ulysses_unpack(const void* src, void* dst, int64_t B, int64_t S_local, int64_t H,
                                    int64_t D, int64_t P, cpattn_dtype dt, cpattn_dir dir,
                                    hipStream_t stream);

/*
 * Batched Ulysses relayout: the same relayout as cpattn_ulysses_pack
 * (cpattn_ulysses_pack_n) or cpattn_ulysses_unpack (cpattn_ulysses_unpack_n)
 * applied to n_tensors tensors of one shape and type in ONE launch, e.g. the
 * Q, K and V shards that go into one all-to-all (first page, "DeepSpeed
 * Ulysses": Q, K and V are exchanged together before attention).  Tensor i is
 * srcs[i] -> dsts[i]; the result equals n_tensors single calls.
 *
 *   srcs, dsts  HOST arrays of n_tensors DEVICE pointers (read during the
 *               call only; the caller keeps ownership of both arrays)
 *   n_tensors   1 .. CPATTN_MAX_RELAYOUT_TENSORS (else CPATTN_E_SHAPE)
 *
 * Every other requirement is the single call's, for each tensor.  No
 * destination may overlap any source or another destination
 * (CPATTN_E_ALIAS); a NULL array or entry is CPATTN_E_NULL.
 */
#define CPATTN_MAX_RELAYOUT_TENSORS 8
cpattn_status cpattn_ulysses_pack_n(const void* const* srcs, void* const* dsts, int64_t n_tensors,
                                    int64_t B, int64_t S_local, int64_t H, int64_t D, int64_t P,
                                    cpattn_dtype dt, cpattn_dir dir, hipStream_t stream);
cpattn_status cpattn_ulysses_unpack_n(const void* const* srcs, void* const* dsts, int64_t n_tensors,
                                      int64_t B, int64_t S_local, int64_t H, int64_t D, int64_t P,
                                      cpattn_dtype dt, cpattn_dir dir, hipStream_t stream);

/*
 * QK-RMSNorm prologue of the attention sample ("TensorRT multi-device
 * attention inference in practice", step 1): per row of D values
 *
 *   y = round16( round16( x * rsqrt(mean(x^2) + eps) * w ) * round16(post_scale) )
 *
 * with the norm evaluated in f32 and round16 the rounding to dt (nearest,
 * ties to even).  The page multiplies Q and K each by (1/D)^(1/4) after the
 * cast; pass that as post_scale, or 1 for the plain RMSNorm (multiplying by 1
 * is exact).
 *
 *   x, y   [rows, D]  dt (BF16 or F16; else CPATTN_E_DTYPE); any layout whose
 *          rows of D are contiguous, e.g. [B, S, H, D] with rows = B*S*H
 *   w      [D]        dt
 *
 * D a power of two in [8, 512] (CPATTN_E_HEADDIM); rows >= 1; eps finite and
 * >= 0, post_scale finite and > 0 and representable after rounding to dt
 * (CPATTN_E_SCALE).  y may be exactly x (in place); any other overlap of y
 * with x or w is CPATTN_E_ALIAS.
 */
cpattn_status cpattn_qk_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int64_t D,
                                float eps, float post_scale, cpattn_dtype dt, hipStream_t stream);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* cpattn_status_string(cpattn_status s);

/* Returns CPATTN_ABI_VERSION of the built library. */
int cpattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H_ */
