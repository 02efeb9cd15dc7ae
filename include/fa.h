/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa.so).
 *
 * The library computes exact attention O = softmax(scale * Q K^T) V and its
 * training gradients without ever writing the N x N score or probability
 * matrices to device memory: the forward walks key/value tiles with running
 * (row max, row sum) statistics, and the backward recomputes the scores tile by
 * tile from Q, K, V and the saved per-row log-sum-exp.
 *
 * Pages this interface follows:
 *   [Training-FA] "Как работает FlashAttention для training (не только
 *                 inference)?" -- aivaro.ru/en/answers/474
 *   [Week-13]     "Неделя 13. GPU и FlashAttention" --
 *                 snula.amonoc.com/course/ru/week-13.html
 *   [FA-guide]    "FlashAttention: IO Farkındalığı ile Hızlı ve Bellek
 *                 Açısından Verimli Tam Dikkat" (reading guide to arXiv
 *                 2205.14135) -- xyznot.com/tr/paper/2205.14135
 *
 * Common conventions for every entry point
 * ----------------------------------------
 *  - Tensors are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees or synchronises; every kernel is enqueued on `stream`
 *    (a hipStream_t; NULL means the default stream) and the call returns
 *    without waiting.
 *  - Q, K, V, O, dO, dQ, dK, dV: [B, H, N, d] contiguous row-major, all of the
 *    same element type `dtype`; 16-byte aligned base pointers.
 *  - LSE: [B, H, N] fp32, natural-log log-sum-exp of each query row's scaled
 *    scores; 4-byte aligned.  -inf for a row that keeps no key.
 *  - block_mask: NULL (dense) or a device array uint8[T][T], T = ceil(N/128),
 *    row-major; entry [i][j] != 0 keeps the 128 x 128 tile of query rows
 *    128i..128i+127 and key rows 128j..128j+127.  One mask is shared by every
 *    (batch, head).  With causal != 0 both restrictions apply.
 *  - causal != 0 keeps key j for query i only when j <= i (self-attention,
 *    N queries against N keys).
 *  - d must be 64 or 128; N >= 1 (any N: the last tile is masked by bounds);
 *    B, H >= 1; N * d and B * H * ceil(N/128) must fit in int32, and one
 *    head's rows, N rounded up to a multiple of 256, times d times the element
 *    size must not exceed 2^32 - 1 bytes (the kernels address a head with
 *    32-bit byte offsets): N <= 8388352 for fp32 at d = 128, N <= 16776960
 *    for bf16 at d = 128.  Larger sizes give FA_ERR_SHAPE.
 *  - scale may be any finite value: [Training-FA] §1 writes
 *    softmax(Q K^T / sqrt(d)) V and [FA-guide] "Problem ve motivasyon" the
 *    unscaled Q K^T, so the scale is a free parameter (1/sqrt(d) is the usual
 *    value; a negative scale flips the sign of every score).
 *  - Outputs must not overlap inputs or each other.
 *  - Validation runs before anything is enqueued; on any error nothing is
 *    written and no kernel is launched.  A launch failure is reported as
 *    FA_ERR_LAUNCH; faults inside a kernel surface, as usual for HIP, at the
 *    caller's next synchronisation.  No C++ exception crosses this interface.
 *  - Calls are stateless and reentrant; results are deterministic (no atomics:
 *    every output element is written by exactly one work-group).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,       /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,      /* B, H or N < 1, a size overflows int32, or one head
                            spans 2^32 bytes or more */
  FA_ERR_HEAD_DIM = 3,   /* d not in {64, 128} */
  FA_ERR_DTYPE = 4,      /* dtype not an fa_dtype value */
  FA_ERR_ALIGN = 5,      /* a tensor pointer is misaligned */
  FA_ERR_WORKSPACE = 6,  /* workspace NULL, misaligned or too small */
  FA_ERR_LAUNCH = 7,     /* the HIP runtime refused a kernel launch */
  FA_ERR_ARG = 8,        /* scale not finite, dropout_p outside [0, 1), or
                            num_splits outside [0, 1024] */
  FA_ERR_ALIAS = 9,      /* an output overlaps an input or another output */
  FA_ERR_SCRATCH = 10,   /* fa_bwd_static: the sizes need more than the
                            library's static scratch holds */
  /* Not statuses: these two give the enum the whole range of int, so that any
     int a caller passes or compares is a valid value of the type. */
  FA_STATUS_INT_MIN_ = -2147483647 - 1,
  FA_STATUS_INT_MAX_ = 2147483647
} fa_status;

typedef enum {
  FA_BF16 = 0,
  FA_FP32 = 1,
  /* Not element types: the whole range of int is a valid value of the type,
     so any int a caller passes reaches the check (FA_ERR_DTYPE). */
  FA_DTYPE_INT_MIN_ = -2147483647 - 1,
  FA_DTYPE_INT_MAX_ = 2147483647
} fa_dtype;

#define FA_MASK_BLOCK 128

/*
 * fa_fwd -- exact attention forward.
 *
 * Computes, for every (b, h) and query row i,
 *   O_i   = sum_j P_ij V_j,  P_ij = exp(s_ij - LSE_i) over kept keys j,
 *   LSE_i = ln sum_{kept j} exp(s_ij),  s_ij = scale * <Q_i, K_j>,
 * tile by tile with running row max and row sum, so S and P stay on chip
 * ([Training-FA] §2.1; [FA-guide] "Yöntem" steps 1-4 and the two-part rule of
 * "Artımsal Softmax Takibi"; [Week-13] Step 2).  Only O and the per-row
 * log-sum-exp are written ([Week-13] Step 2 keeps the logsumexp for the
 * backward).  Arithmetic: bf16 (or fp32) operands, fp32 accumulation and
 * statistics; P is rounded to the operand type before the P V product.
 * A row with no kept key gets O_i = 0 and LSE_i = -inf.
 *
 *   Q, K, V   in : [B,H,N,d] dtype
 *   O         out: [B,H,N,d] dtype (overwritten)
 *   LSE       out: [B,H,N] fp32 (overwritten)
 */
fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int B, int H, int N, int d, float scale, int causal,
                 const unsigned char* block_mask, fa_dtype dtype, void* stream);

/*
 * fa_fwd_workspace_bytes / fa_fwd_ws -- the forward with an optional
 * workspace.  In bf16, a shape with fewer than 256 query blocks (of 256 rows
 * at d = 128 without a block mask, else of 128 rows; e.g. one head of a long
 * sequence) leaves most of the GPU idle while its last block walks every
 * key; given a workspace of at least fa_fwd_workspace_bytes bytes,
 * fa_fwd_ws cuts each block's 64-key tiles into runs (at most 8, at least 8
 * tiles each), one work-group per run, each writing its normalised O and its
 * LSE in fp32 to the workspace (O: runs * B*H*N*d * 4 bytes, then LSE:
 * runs * B*H*N * 4 bytes), and a second kernel merges the runs per row in
 * run order with the two-part rule ([FA-guide] "Artımsal Softmax Takibi"):
 * deterministic, equal to fa_fwd's result up to rounding.
 * fa_fwd_workspace_bytes (the larger of the unmasked and block-masked
 * plans) returns 0 when no split applies; then, and with a smaller or NULL
 * workspace (workspace_bytes 0), fa_fwd_ws is fa_fwd.
 * The workspace is caller-owned device memory, 16-byte aligned, not
 * overlapping any argument (FA_ERR_WORKSPACE / FA_ERR_ALIGN / FA_ERR_ALIAS);
 * other arguments and errors as for fa_fwd.
 */
size_t fa_fwd_workspace_bytes(int B, int H, int N, int d);
fa_status fa_fwd_ws(const void* Q, const void* K, const void* V, void* O, float* LSE,
                    int B, int H, int N, int d, float scale, int causal,
                    const unsigned char* block_mask, fa_dtype dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * fa_bwd_workspace_bytes -- size of the scratch buffer fa_bwd uses: one fp32
 * per query row (D_i = sum_k dO_ik O_ik), i.e. 4 * B * H * N bytes, so the
 * backward's extra memory is O(N) ([FA-guide] "Karmaşıklık Analizi") --
 * plus, for shapes whose blocks would fill fewer than the GPU's 256 compute
 * units (B * H * ceil(N/128) < 256, e.g. one head of a long sequence), the
 * fp32 partials of the split passes (see fa_bwd_splits): D rounded up to 256
 * bytes, then 2 * s_kv * B * H * N * d * 4 bytes when s_kv > 1, then
 * s_q * B * H * N * d * 4 bytes when s_q > 1.  Any workspace of at least
 * 4 * B * H * N bytes is accepted; with less than this size the passes run
 * unsplit.  The size does not depend on the element type.  Returns 0 for
 * sizes that fa_bwd rejects with FA_ERR_SHAPE for either element type.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd_splits -- how fa_bwd, fa_bwd_dropout and fa_bwd_gqa divide the work
 * of the backward for a shape, given a workspace of the preferred size.
 * Outputs (host pointers, non-NULL):
 *   *dkdv_split  work-groups per (key/value head, 128-key block) of the dK/dV
 *                pass: the group's query heads (grouped heads, as described
 *                at fa_bwd_gqa) or, with one query head per key/value head,
 *                runs of its 128-row query tiles;
 *   *dq_split    work-groups per (query head, 128-row query block) of the dQ
 *                pass, each taking a run of its 64-key tiles.
 * Splits apply to bf16 only, where fewer than 256 blocks would run: a split
 * pass writes fp32 partials into the workspace and a reduction kernel adds
 * them in a fixed order, so results stay deterministic (but differ in
 * rounding from the unsplit passes').  At most 8 runs, at least 4 query tiles
 * (dK/dV) or 8 key tiles (dQ) per run.  The phase entry points
 * (fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_dq_and_d) and
 * fa_bwd_static never split.
 * Errors: FA_ERR_NULL, and the shape checks of fa_bwd_gqa (Hq = H, Hkv = H
 * for the plain backward).
 */
fa_status fa_bwd_splits(int B, int Hq, int Hkv, int N, int d, fa_dtype dtype,
                        int* dkdv_split, int* dq_split);

/*
 * fa_bwd -- gradients of sum(O * dO) with respect to Q, K and V.
 *
 * Recomputes S and P block by block from Q, K and the saved LSE instead of
 * reading a stored P ([Training-FA] §3 and §3.1; [Week-13] Step 2), using
 * the closed form of the chain rule through softmax:
 *   D_i = sum_k dO_ik O_ik,  dV = P^T dO,  dP = dO V^T,
 *   dS = P * (dP - D 1^T),   dQ = scale * dS K,  dK = scale * dS^T Q.
 * Two kernels run in order on `stream`: a pass that is parallel over query
 * blocks, forms D from the O and dO rows it holds (writing it to the
 * workspace) and accumulates dQ on chip (no atomics), then a pass that is
 * parallel over key blocks, reads D and accumulates dK and dV on chip.
 * Tiles dropped by causality or the block mask are skipped in both passes.
 *
 *   Q, K, V, O, dO  in : [B,H,N,d] dtype; O and LSE from fa_fwd with the
 *                        same Q, K, V, scale, causal and block_mask
 *   LSE             in : [B,H,N] fp32
 *   dQ, dK, dV      out: [B,H,N,d] dtype (overwritten, not accumulated)
 *   workspace       scratch of at least fa_bwd_workspace_bytes(B,H,N,d)
 *                   bytes, 16-byte aligned, caller-owned; its contents are
 *                   overwritten and need no initialisation.
 */
fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O,
                 const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                 int B, int H, int N, int d, float scale, int causal,
                 const unsigned char* block_mask, fa_dtype dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * The phases of the backward, callable one by one: fa_bwd_preprocess, then
 * fa_bwd_dkdv and fa_bwd_dq give results bit-identical to fa_bwd's (whose
 * dQ pass, fa_bwd_dq_and_d below, forms D itself, adding the same products
 * in the same order as fa_bwd_preprocess).  The dK/dV and dQ passes only
 * read what the preprocess wrote, so a caller may enqueue them on two
 * streams that both wait for the preprocess.  Arguments have the meaning,
 * layout and checks given for fa_bwd.
 *
 * fa_bwd_preprocess: workspace[i] = D_i = sum_k dO_ik O_ik (fp32), the
 *   row term of dS = P * (dP - D 1^T).
 * fa_bwd_dkdv: dK = scale * dS^T Q and dV = P^T dO, one work-group per 128
 *   keys, recomputing S and P per query tile ([Training-FA] §3.1).
 * fa_bwd_dq: dQ = scale * dS K, one work-group per 128 queries, recomputing
 *   S, P and dP per key tile; no atomics.
 */
fa_status fa_bwd_preprocess(const void* O, const void* dO, int B, int H, int N, int d,
                            fa_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream);
fa_status fa_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                      const float* LSE, void* dK, void* dV, int B, int H, int N, int d,
                      float scale, int causal, const unsigned char* block_mask,
                      fa_dtype dtype, const void* workspace, size_t workspace_bytes,
                      void* stream);
fa_status fa_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
                    const float* LSE, void* dQ, int B, int H, int N, int d, float scale,
                    int causal, const unsigned char* block_mask, fa_dtype dtype,
                    const void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_dq_and_d -- fa_bwd's own first kernel: the dQ pass of fa_bwd_dq
 * that also forms D_i = sum_k dO_ik O_ik from the O and dO rows it holds
 * (instead of reading it) and writes it to the workspace, bit-identical to
 * what fa_bwd_preprocess writes.  fa_bwd is exactly fa_bwd_dq_and_d, then
 * fa_bwd_dkdv, on one stream.  Arguments as for fa_bwd; the workspace
 * (at least 4 * B * H * N bytes) is written, not read.
 */
fa_status fa_bwd_dq_and_d(const void* Q, const void* K, const void* V, const void* O,
                          const void* dO, const float* LSE, void* dQ, int B, int H, int N,
                          int d, float scale, int causal, const unsigned char* block_mask,
                          fa_dtype dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * fa_bwd_static -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same gradients, the same kernels and checks, but no
 * workspace argument.  The row term D goes to a static device array of
 * FA_STATIC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends; the call allocates nothing.  It needs
 * 4 * B * H * N <= FA_STATIC_SCRATCH_BYTES (else FA_ERR_SCRATCH, nothing
 * enqueued).  The device address of the array is looked up on the first call
 * on each device (with that device current); a failed lookup gives
 * FA_ERR_LAUNCH.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams without ordering between them)
 * race on it.  Its contents need no initialisation (every value of D is
 * written before it is read).
 */
#define FA_STATIC_SCRATCH_BYTES 4194304
fa_status fa_bwd_static(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                        int B, int H, int N, int d, float scale, int causal,
                        const unsigned char* block_mask, fa_dtype dtype, void* stream);

/*
 * fa_fwd_dropout / fa_bwd_dropout -- fa_fwd and fa_bwd with dropout on the
 * attention probabilities, fused into the same kernels (the FlashAttention
 * reading guide, xyznot.com/tr/paper/2205.14135, "Temel fikirler", lists
 * dropout among the operations fused with the matrix products, masking and
 * softmax).  With keep mask Z and M = Z / (1 - dropout_p):
 *   O = (P * M) V;  LSE is that of the undropped P (unchanged by dropout);
 *   dV = (P * M)^T dO,  dP = (dO V^T) * M,  D_i = sum_k dO_ik O_ik,
 *   dS = P * (dP - D 1^T),  dQ = scale * dS K,  dK = scale * dS^T Q.
 * Z is never stored: both calls regenerate it.  Element (i, j) (query i,
 * key j) of head bh = b*H + h takes word (j mod 4) of Philox4x32 with 10
 * rounds (Salmon, Moraes, Dror, Shaw, SC 2011) on counter (j / 4, i / 2, bh, 0)
 * with key (seed mod 2^32, seed / 2^32) -- its low 16 bits for even i, its
 * high 16 bits for odd i -- and is kept iff that value is
 * >= min(floor(dropout_p * 2^16), 2^16 - 1) (one call covers two queries and
 * four keys; the drop rate is within 2^-16 of dropout_p, the kept
 * probabilities are scaled by 1 / (1 - dropout_p)).  fa_bwd_dropout must get
 * the dropout_p and
 * seed that fa_fwd_dropout got (and its O and LSE).  Other arguments as for
 * fa_fwd / fa_bwd; dropout_p must lie in [0, 1) (else FA_ERR_ARG).
 */
fa_status fa_fwd_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE,
                         int B, int H, int N, int d, float scale, int causal,
                         const unsigned char* block_mask, float dropout_p,
                         unsigned long long seed, fa_dtype dtype, void* stream);
fa_status fa_bwd_dropout(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                         int B, int H, int N, int d, float scale, int causal,
                         const unsigned char* block_mask, float dropout_p,
                         unsigned long long seed, fa_dtype dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * fa_fwd_gqa / fa_bwd_gqa -- fa_fwd and fa_bwd with grouped key/value heads
 * (GQA; MQA when Hkv = 1): query heads h = kvh*G .. kvh*G+G-1, G = Hq / Hkv,
 * all attend with key/value head kvh (the week-13 page,
 * snula.amonoc.com/course/ru/week-13.html, names GQA: one key/value head per
 * group of query heads).  The forward and dQ are those of fa_fwd / fa_bwd per
 * query head; a shared head's dK and dV are the sums over its G query heads,
 * accumulated on chip by one work-group per 128 keys that walks the tiles of
 * all G heads (no atomics; deterministic).
 *
 *   Q, O, dO, dQ : [B, Hq, N, d] dtype;  LSE: [B, Hq, N] fp32
 *   K, V, dK, dV : [B, Hkv, N, d] dtype (dK, dV overwritten)
 *   workspace    : at least fa_bwd_gqa_workspace_bytes(B, Hq, Hkv, N, d) bytes
 * Hq must be a multiple of Hkv (FA_ERR_SHAPE otherwise); other arguments and
 * checks as for fa_fwd / fa_bwd (with H = Hq).  Hkv = Hq gives exactly
 * fa_fwd / fa_bwd.  When B * Hkv * ceil(N/128) is small (under 512 work-groups)
 * a group's query heads are divided among up to G work-groups that each write
 * an fp32 partial dK, dV into the workspace, and a third kernel adds the
 * partials in a fixed order (still deterministic).
 *
 * fa_bwd_gqa_workspace_bytes: 4 * B * Hq * N bytes for D, plus, when the dK/dV
 * work is divided, 2 * splits * B * Hkv * N * d * 4 bytes of partials; 0 for
 * sizes fa_bwd_gqa would reject.
 */
size_t fa_bwd_gqa_workspace_bytes(int B, int Hq, int Hkv, int N, int d);
fa_status fa_fwd_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     const unsigned char* block_mask, fa_dtype dtype, void* stream);
fa_status fa_bwd_gqa(const void* Q, const void* K, const void* V, const void* O,
                     const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     const unsigned char* block_mask, fa_dtype dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * fa_fwd_fp8 -- attention forward on FP8 inputs, both products on the gfx950
 * FP8 matrix cores (FlashAttention-3 runs its forward in FP8: [Training-FA],
 * the list of versions; [Week-13], the note on FA2 and FA3).
 *
 * Values are OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; largest magnitude 448) with fp32 block scales: the value of a code c
 * of Q (K) in row block t = r / 128 of head (b, h) is E4M3(c) *
 * q_scale[b][h][t] (k_scale), of V E4M3(c) * v_scale[b][h].  The result is
 * attention on those values (O, LSE as for fa_fwd); the probabilities are
 * rounded to E4M3 for the P V product (P~ = 2^8 e^(s - m) <= 256, m the
 * running row max), the row sums are not.
 *
 *   Q8, K8    in : [B, H, N, d] uint8 codes
 *   Vt8       in : [B, H, d, N] uint8 codes (V transposed); all codes finite
 *   q_scale, k_scale in: [B, H, ceil(N/128)] fp32 (> 0);  v_scale in: [B, H] fp32
 *   O         out: [B, H, N, d] bf16;  LSE out: [B, H, N] fp32
 * N must be a multiple of 16 (FA_ERR_SHAPE otherwise); other checks as for
 * fa_fwd.
 */
fa_status fa_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, const float* q_scale,
                     const float* k_scale, const float* v_scale, void* O, float* LSE, int B,
                     int H, int N, int d, float scale, int causal,
                     const unsigned char* block_mask, void* stream);

/*
 * fa_decode -- attention of a few new query rows against a key/value cache,
 * with grouped key/value heads (inference decode; the week-13 page's note on
 * decode attention and GQA, snula.amonoc.com/course/ru/week-13.html).
 *
 * For batch entry b, query head h (cache head kvh = h / (Hq / Hkv)) and new
 * query row i:
 *   O_bhi   = sum_j P_j V[b, kvh, j],  P_j = exp(s_j - LSE_bhi) over visible j,
 *   LSE_bhi = ln sum_{visible j} exp(s_j),  s_j = scale * <Q_bhi, K[b, kvh, j]>,
 * where key j is visible iff j < L_b and, with causal != 0, j <= L_b - Nq + i
 * (the Nq new tokens are the last Nq positions of the sequence).  A row with
 * no visible key gets O = 0 and LSE = -inf.  The keys of each (b, kvh) are
 * cut into chunks handled by separate work-groups (each cache byte is read
 * once and serves the Hq / Hkv query heads of its group); the chunks' partial
 * (LSE, O) are merged with the two-part rule of [FA-guide] "Artımsal Softmax
 * Takibi" by a second kernel.  Arithmetic as in fa_fwd.
 *
 *   Q        in : [B, Hq, Nq, d] dtype
 *   K, V     in : [B, Hkv, Nkv, d] dtype (cache rows at or past L_b are never read)
 *   seqlens  in : device int32[B] with L_b in [0, Nkv] (values outside are
 *                 clamped to that range), or NULL: every L_b = Nkv
 *   O        out: [B, Hq, Nq, d] dtype (overwritten)
 *   LSE      out: [B, Hq, Nq] fp32 (overwritten)
 *   num_splits    0: the library picks the number of key chunks; n >= 1: at
 *                 most n chunks (n <= 1024)
 *   workspace     scratch of at least fa_decode_workspace_bytes(...) bytes
 *                 (0 when a single chunk is used: then workspace may be NULL),
 *                 16-byte aligned, caller-owned, contents overwritten.
 *
 * Hq must be a multiple of Hkv (FA_ERR_SHAPE otherwise); B, Hq, Hkv, Nq,
 * Nkv >= 1; Nkv * d and B * Hq * Nq * d must fit in int32, and one cache
 * head (Nkv rows) and one group's Hq / Hkv * Nq query rows obey the 2^32-byte
 * head bound above; seqlens 4-byte aligned.  Other conventions as above.
 */
fa_status fa_decode(const void* Q, const void* K, const void* V, const int* seqlens, void* O,
                    float* LSE, int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale,
                    int causal, int num_splits, fa_dtype dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * fa_decode_num_splits -- the number of key chunks fa_decode uses for these
 * sizes and num_splits (1: no merge kernel and no workspace); 0 for sizes
 * fa_decode would reject.
 * fa_decode_workspace_bytes -- the workspace fa_decode needs for them:
 * (d + 1) * 4 bytes per query row and chunk when more than one chunk is used,
 * else 0 (also 0 for rejected sizes).
 */
int fa_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int num_splits);
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int d,
                                 int num_splits);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* fa_status_str(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
