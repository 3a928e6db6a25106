/*
 * dg.h - C ABI of libdg: the hot path of one block-diffusion denoising step on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM"
 *        (agentlenshq.com summary of the vLLM integration)
 *   [P2] "DiffusionGemma 개발자 가이드" (molayo1419.me retelling of the developer guide)
 *   [P3] "DiffusionGemma u vLLM: prvi diskretni difuzijski model od 26 milijardi
 *        parametara integriran u produkcijsko okruženje" (24-ai.news)
 *
 * The three calls follow the split of the per-model hooks in [P1] section
 * "ModelState 인터페이스" and [P3] section "Integracija u vLLM infrastrukturu":
 *   dg_attn_mixed      - attention with a causal/bidirectional switch per request
 *                        (the prepare_attn hook and the attention backend);
 *   dg_sampler_step    - the DiffusionSampler's denoise step (the custom_sampler hook);
 *   dg_selfcond_embed  - the self-conditioning average (the self-conditioning part
 *                        of the prepare_inputs hook).
 * Per-request state (canvas, previous argmax, stable count) lives in caller
 * buffers, standing in for the add_request/remove_request lifecycle.
 *
 * Conventions shared by every call:
 *   - Pointers marked "device" are device (HBM) addresses; "host" ones are read on
 *     the host during the call and may be freed when it returns.
 *   - The caller owns every buffer, the workspace included (size it with the
 *     matching dg_*_workspace_size). The library never allocates, frees or
 *     synchronises; every call is asynchronous on `stream` (a hipStream_t, NULL for
 *     the default stream) and performs no host<->device copy.
 *   - Every argument is validated before anything is launched. On any error the
 *     call launches nothing, writes no output, returns a non-zero dg_status and
 *     leaves a message for dg_last_error() (thread-local). Launch failures return
 *     DG_ERR_HIP; faults inside a kernel surface at the caller's next synchronisation.
 *   - Results are deterministic: the same inputs, seeds and steps give bit-identical
 *     outputs (no floating-point atomics; every split is merged in a fixed order).
 *   - Row-major layouts; the last dimension is contiguous. Device buffers must be
 *     16-byte aligned.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_ABI_VERSION 3
#define DG_MAX_SEQS 64      /* requests per dg_attn_mixed call */
#define DG_MAX_REQS 64      /* requests per dg_sampler_step call */
#define DG_MAX_CANVAS 1024  /* positions per sampler request */
#define DG_PROB_BLOCK 8192  /* vocabulary entries per scale of a block-scaled probability matrix */

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = 1, /* an argument breaks a documented rule */
  DG_ERR_UNSUPPORTED = 2, /* valid in principle but not built (e.g. head_dim) */
  DG_ERR_WORKSPACE = 3,   /* workspace missing or smaller than dg_*_workspace_size */
  DG_ERR_HIP = 4          /* the HIP runtime refused a launch */
} dg_status;

typedef enum { DG_F32 = 0, DG_BF16 = 1 } dg_dtype;

/* Per-request attention mode ([P1] sections "듀얼 모드 운영" and
 * "동적 퍼-시퀀스 인과적 어텐션"): prefill and commit are causal ("encoder mode"),
 * denoising is bidirectional ("decoder mode"). */
typedef enum { DG_CAUSAL = 0, DG_BIDIR = 1 } dg_mode;

/* ------------------------------------------------------------------------------
 * dg_attn_mixed: masked softmax attention for a batch of requests in mixed modes.
 *
 * Request r owns query rows [q_start, q_start + num_q) of q/out/lse and key rows
 * [kv_start, kv_start + prefix_len + num_q) of k/v: the first prefix_len rows are
 * its committed KV cache, the last num_q rows are this call's tokens (the canvas,
 * a commit or a prefill), whose K/V the caller has already written. New token i
 * sits at position p = prefix_len + i and attends to keys j of its own request with
 *     lo <= j <= hi,  lo = (window < 0) ? 0 : max(0, p - window),
 *     hi = CAUSAL ? p : (window < 0 ? prefix_len + num_q - 1
 *                                   : min(prefix_len + num_q - 1, p + window)).
 * So a causal request in a sliding-window layer sees the `window` tokens before
 * it plus itself, and a bidirectional one up to `window` on each side, 2W+1 keys
 * ([P1] section "대칭 슬라이딩 윈도우 어텐션"; [P3] decoder mode with +-W windows).
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) (grouped heads).
 *   out[t, h, :] = sum_j softmax_j(scale * <q[t,h], k[j,g]>) * v[j, g, :]
 *   lse[t, h]    = log sum_j exp(scale * <q[t,h], k[j,g]>)      (natural log)
 *
 * Paged K/V (block_size > 0). A committed block is appended to the request's cache
 * and the canvas is redrafted every step ([P1] sections "샘플링 루프와 엔트로피 경계
 * 디노이징" and "ModelState 인터페이스"; [P3] section "Integracija u vLLM
 * infrastrukturu", which keeps vLLM's paged cache). In this mode k and v are pools of
 * total_kv / block_size blocks of block_size rows, and key j of request r (cache and
 * new tokens alike) sits at pool row
 *     block_table[kv_start + j / block_size] * block_size + j % block_size,
 * so kv_start is the index of the request's first table entry. The result is the one
 * the contiguous layout gives for the same key rows, bit for bit. Table entries are
 * device data and are not checked on the host: an entry outside [0, total_kv /
 * block_size) gives unspecified results for that request (the kernels clamp it, so
 * they never read outside the pools). dg_kv_write fills the pools.
 *
 * FP8 K/V (kv_fp8 = 1). The measured model runs in FP8 ([P1] section "성능 및
 * 양자화"; [P3] section "Izmjerene performanse"). In this mode k and v hold one byte
 * per element, a code of the OCP 8-bit floating point format E4M3 (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent 0 subnormal; S.1111.111 NaN; largest
 * finite 448), in the same layouts as above (contiguous or paged), and
 *   k[j, g, :] = code * k_scale,   v[j, g, :] = code * v_scale
 * enter the formulas above. q and out stay bf16 (dtype must be DG_BF16); the codes
 * are widened to bf16 exactly and the products accumulate in fp32; k_scale joins the
 * score scale and v_scale the output normalisation, both in fp32.
 * ------------------------------------------------------------------------------ */
typedef struct {
  int32_t q_start, num_q, kv_start, prefix_len, mode; /* mode: dg_mode */
} dg_seq;

typedef struct {
  int32_t num_seqs;             /* 1..DG_MAX_SEQS */
  const dg_seq* seqs;           /* host array [num_seqs]; query ranges must not overlap */
  int32_t window;               /* -1: global layer; W >= 0: sliding window */
  int32_t num_q_heads;          /* Hq >= 1 */
  int32_t num_kv_heads;         /* Hkv >= 1, Hq % Hkv == 0, Hq / Hkv in {1,2,4,8,16,32} (else DG_ERR_UNSUPPORTED) */
  int32_t head_dim;             /* D in {64, 128, 256} */
  float scale;                  /* 0 => 1/sqrt(head_dim) */
  int32_t dtype;                /* dg_dtype of q, k, v and out */
  int64_t total_q;              /* rows of q/out/lse: every q range must fit */
  int64_t total_kv;             /* rows of k/v: every kv range must fit */
  const void* q;                /* device [total_q, Hq, D] */
  const void* k;                /* device [total_kv, Hkv, D] */
  const void* v;                /* device [total_kv, Hkv, D] */
  void* out;                    /* device [total_q, Hq, D], dtype; rows outside every request untouched */
  float* lse;                   /* device [total_q, Hq] fp32, or NULL */
  int32_t kv_chunk;             /* keys per split-KV chunk: 0 = library's choice, else a multiple of 64 */
  void* workspace;              /* device, >= dg_attn_workspace_size(args) bytes (may be NULL if that is 0) */
  size_t workspace_bytes;
  int32_t block_size;           /* 0: contiguous K/V; else a power of two >= 64, dividing total_kv (paged) */
  const int32_t* block_table;   /* device [block_table_len] int32 when block_size > 0, else ignored */
  int64_t block_table_len;      /* every request needs kv_start + ceil((prefix_len + num_q) / block_size) <= this */
  int32_t kv_fp8;               /* 0: k and v are in dtype; 1: k and v hold E4M3 codes, dtype must be DG_BF16
                                   (else DG_ERR_UNSUPPORTED); other values and bad scales: DG_ERR_INVALID_ARG */
  float k_scale;                /* kv_fp8: finite, > 0; ignored otherwise */
  float v_scale;                /* kv_fp8: finite, > 0; ignored otherwise */
} dg_attn_args;

dg_status dg_attn_mixed(const dg_attn_args* args, void* stream);
/* Workspace the call needs for these arguments (split-KV partials and the work
 * list). Pure host; 0 means none. Returns (size_t)-1 if the arguments are invalid. */
size_t dg_attn_workspace_size(const dg_attn_args* args);

/* ------------------------------------------------------------------------------
 * dg_sampler_step: one denoise step of the DiffusionSampler over canvas rows
 * ([P1] section "샘플링 루프와 엔트로피 경계 디노이징"; [P3] section
 * "Mehanizam odlučivanja o gotovim tokenima"; re-noising of unaccepted positions,
 * [P2] sections "아키텍처 (The Architecture)" and "Diffusion에 스도쿠가 흥미로운 이유").
 *
 * Row statistics, for each row i of logits (every row 0..num_rows-1):
 *   row_max[i] = max_v l[i,v];  argmax[i] = lowest v with l[i,v] = row_max[i];
 *   row_sum[i] = sum_v exp(l[i,v] - row_max[i]);  p = exp(l - row_max) / row_sum;
 *   entropy[i] = -sum_v p_v ln p_v (nats, >= 0);
 *   conf[i]    = -entropy[i] (DG_CONF_NEG_ENTROPY) or 1/row_sum, the largest
 *                probability (DG_CONF_MAX_PROB).
 * Per request r (rows [row_start, row_start + num_rows), position j = row - row_start):
 *   cand    = first token whose cumulative probability exceeds u, u = Philox4x64-10
 *             24-bit uniform for key (seed, 0), counter (step, j, 0, 0);
 *   accept  = the longest run of positions, most confident first (ties: lower j
 *             first), whose entropy total stays <= budget, and at least min_accept
 *             positions; totals are exact integer sums of floor(entropy * 2^40);
 *   canvas  = accept ? cand : converged ? argmax : renoise ? token : canvas, where the
 *             token is floor(hi32(x0) * vocab / 2^32) of Philox counter (step, j, 1, 0);
 *   stable_count = (step > 0 and argmax == prev_argmax at every position)
 *                  ? stable_count + 1 : 0;
 *   mean_entropy = sum floor(entropy * 2^40) / 2^40 / num_rows;
 *   converged    = DG_CONV_AND: (stable_count >= stable_k and mean < tau) or step + 1 >= step_limit
 *                  DG_CONV_OR:  stable_count >= stable_k or mean < tau or step + 1 >= step_limit
 *                  (mean < tau is tested exactly in the 2^-40 fixed point);
 *   prev_argmax  = argmax.
 * With DG_ENTROPY_IN the call reads `entropy` (and, for DG_CONF_MAX_PROB, `conf`)
 * instead of writing them, so a selection can be replayed on given entropies.
 * Block-scaled probabilities (optional, for dg_selfcond_embed): with probs and
 * probs_scale set, the call also writes w[i,v] (logits dtype) and s[i,b] (fp32) with
 *   softmax(l[i,:])[v] = w[i,v] * s[i, v / DG_PROB_BLOCK]   (w rounded to the dtype),
 * w = exp(l - max over the chunk of the row that holds v), s = the chunk's exp(max - row_max) / row_sum.
 * With DG_INIT_CANVAS the call only starts a block: canvas = Philox token from
 * counter (step, j, 2, 0), prev_argmax = -1, stable_count = 0, converged = 0,
 * num_accepted = 0; logits are not read.
 * The step splits in two calls with the same arguments, for a caller that overlaps
 * the selection with work that needs only the row outputs (self-conditioning reads the
 * probabilities): DG_SKIP_SELECT computes the row statistics, candidates and
 * probabilities and leaves accept, canvas, prev_argmax and the per-request state
 * untouched; DG_SELECT_ONLY then runs the selection alone on the entropy, conf, argmax
 * and cand that call wrote (logits and the workspace are not used). The pair gives
 * exactly the results of one call without either flag.
 * Precondition: every logits row has at least one finite value (-inf means p = 0).
 * ------------------------------------------------------------------------------ */
#define DG_CONF_NEG_ENTROPY 0
#define DG_CONF_MAX_PROB 1
#define DG_CONV_AND 0
#define DG_CONV_OR 1
#define DG_ENTROPY_IN 1u
#define DG_INIT_CANVAS 2u
#define DG_SKIP_SELECT 4u
#define DG_SELECT_ONLY 8u

typedef struct {
  int32_t row_start, num_rows; /* rows of this request's canvas; 1..DG_MAX_CANVAS rows */
  uint64_t seed;               /* Philox key word 0 */
  int32_t step;                /* denoise step index within the block, >= 0 */
  int32_t reserved;            /* must be 0 */
} dg_sreq;

typedef struct {
  int32_t num_reqs;            /* 1..DG_MAX_REQS */
  const dg_sreq* reqs;         /* host array; request row ranges must not overlap */
  int32_t num_rows;            /* M: rows of logits and of every [M] buffer */
  int32_t vocab;               /* V >= 1 */
  int32_t dtype;               /* dg_dtype of logits */
  const void* logits;          /* device [M, ld] */
  int64_t ld;                  /* row stride of logits in elements, >= V, multiple of 8 */
  float budget;                /* entropy budget in nats, finite, >= 0 */
  int32_t min_accept;          /* >= 0 */
  int32_t conf_mode;           /* DG_CONF_* */
  int32_t renoise;             /* 1: re-noise unaccepted positions; 0: keep their token */
  int32_t stable_k;            /* >= 1 */
  float tau;                   /* mean-entropy threshold, finite, >= 0 */
  int32_t step_limit;          /* >= 1 */
  int32_t combine;             /* DG_CONV_* */
  uint32_t flags;              /* DG_ENTROPY_IN | DG_INIT_CANVAS | DG_SKIP_SELECT | DG_SELECT_ONLY */
  float* entropy;              /* device [M] (input with DG_ENTROPY_IN) */
  float* conf;                 /* device [M] (input with DG_ENTROPY_IN and DG_CONF_MAX_PROB) */
  float* row_max;              /* device [M] */
  float* row_sum;              /* device [M] */
  int32_t* argmax;             /* device [M] */
  int32_t* cand;               /* device [M]; -1 for rows outside every request */
  uint8_t* accept;             /* device [M] (0/1) */
  int32_t* canvas;             /* device [M], in/out */
  int32_t* prev_argmax;        /* device [M], in/out */
  int32_t* stable_count;       /* device [num_reqs], in/out */
  int32_t* num_accepted;       /* device [num_reqs] */
  int32_t* converged;          /* device-accessible [num_reqs] (0/1), write-only: device memory, or pinned
                                  host memory (hipHostMalloc, coherent) that the host reads once the
                                  call's work has completed, with no copy on the stream */
  float* mean_entropy;         /* device [num_reqs] */
  void* probs;                 /* device [M, ldq] (logits dtype) or NULL: block-scaled probabilities w */
  int64_t ldq;                 /* row stride of probs in elements, >= V, multiple of 8 */
  float* probs_scale;          /* device [M, ceil(V / DG_PROB_BLOCK)] or NULL (set both or neither) */
  void* workspace;             /* device, >= dg_sampler_workspace_size(args) bytes */
  size_t workspace_bytes;
  int32_t* step_counter;       /* device [num_reqs] int32 (4-byte aligned, else DG_ERR_INVALID_ARG), caller-owned,
                                  or NULL (then reqs[r].step is the step). When set,
                                  request r's step is read from step_counter[r] when the kernels run and
                                  reqs[r].step is ignored; DG_INIT_CANVAS draws with reqs[r].step as
                                  before and sets step_counter[r] = 0; a call that runs the selection
                                  (no DG_SKIP_SELECT) stores step + 1 there after it. So one recorded
                                  sequence of calls (a HIP graph of a denoise step) replays as
                                  successive steps. */
} dg_sampler_args;

dg_status dg_sampler_step(const dg_sampler_args* args, void* stream);
size_t dg_sampler_workspace_size(const dg_sampler_args* args);

/* dg_sampler_step_noalloc: dg_sampler_step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, validation, kernels and results as dg_sampler_step, except that
 * args->workspace and args->workspace_bytes are ignored: the workspace is a static device
 * array of DG_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends. The call allocates and frees nothing. A call whose
 * dg_sampler_workspace_size exceeds DG_NOALLOC_SCRATCH_BYTES returns DG_ERR_WORKSPACE
 * and launches nothing (4 MiB holds about 1800 rows at a 262144-entry bf16 vocabulary).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (on different streams, or from different threads without ordering) race and give
 * undefined results. The array keeps the last call's contents; a call reads only what it
 * wrote itself. The first call on each device looks up the array's device address
 * (hipGetSymbolAddress) with that device current; a failure there returns DG_ERR_HIP. */
#define DG_NOALLOC_SCRATCH_BYTES (4u << 20)
dg_status dg_sampler_step_noalloc(const dg_sampler_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * dg_selfcond_embed: the probability-weighted average of the token embeddings
 * ([P1] section "안정성을 위한 셀프 컨디셔닝"; [P3] section
 * "Mehanizam odlučivanja o gotovim tokenima"):
 *   out[i, :] = sum_v p[i, v] * embed[v, :]
 * p is given in one of three forms:
 *   - probabilities (row_max, row_sum and p_scale NULL);
 *   - logits with the sampler's row statistics, p = exp(l - row_max[i]) / row_sum[i]
 *     (row_max and row_sum set);
 *   - block-scaled, p[i,v] = w[i,v] * p_scale[i, v / DG_PROB_BLOCK], as dg_sampler_step
 *     writes it (p holds w, p_scale set).
 * Products are accumulated in fp32; out has the input dtype.
 * ------------------------------------------------------------------------------ */
typedef struct {
  int32_t M, V, d;             /* M >= 1; V >= 1; d a multiple of 128 */
  int32_t dtype;               /* dg_dtype of p/logits, embed and out */
  const void* p;               /* device [M, ldp]: probabilities, or logits with row stats */
  int64_t ldp;                 /* >= V, multiple of 8 */
  const float* row_max;        /* device [M] or NULL */
  const float* row_sum;        /* device [M] or NULL (set both or neither) */
  const float* p_scale;        /* device [M, ceil(V / DG_PROB_BLOCK)] or NULL; excludes row_max */
  const void* embed;           /* device [V, lde] */
  int64_t lde;                 /* >= d, multiple of 8 */
  void* out;                   /* device [M, ldo], dtype */
  int64_t ldo;                 /* >= d */
  void* workspace;             /* device, >= dg_selfcond_workspace_size(args) bytes */
  size_t workspace_bytes;
} dg_selfcond_args;

dg_status dg_selfcond_embed(const dg_selfcond_args* args, void* stream);
size_t dg_selfcond_workspace_size(const dg_selfcond_args* args);

/* ------------------------------------------------------------------------------
 * dg_kv_write: write new K/V rows into paged pools (the layout dg_attn_mixed reads
 * with block_size > 0). This is the cache side of a request's life ([P1] sections
 * "샘플링 루프와 엔트로피 경계 디노이징" and "ModelState 인터페이스"): a prefill or a
 * committed block appends its rows after the request's cache, and a canvas draft
 * rewrites the same positions at every denoise step.
 * For request r, row src_start + i of k_new/v_new (i < num) goes to the request's key
 * position pos + i, i.e. pool row
 *     block_table[table_start + (pos + i) / block_size] * block_size + (pos + i) % block_size.
 * Rows of the pools that no request writes are left untouched. Target rows of
 * different requests must not overlap (they would race). Table entries are not
 * checked on the host; the kernel skips a row whose entry lies outside the pool.
 * FP8 pools (pool_fp8 = 1): the pools hold E4M3 codes, one byte per element (the
 * format dg_attn_mixed reads with kv_fp8 = 1), and each new value x (in dtype) is
 * quantized: y = x * r in fp32, r = 1 / scale rounded to fp32 on the host, y clamped
 * to [-448, 448], then the nearest E4M3 value, ties to the even code (NaN stays NaN).
 * ------------------------------------------------------------------------------ */
typedef struct {
  int32_t src_start;            /* first row of k_new / v_new */
  int32_t num;                  /* rows to write, >= 0 */
  int32_t table_start;          /* index of the request's first block_table entry */
  int32_t pos;                  /* key position of the first row within the request, >= 0 */
} dg_kv_seq;

typedef struct {
  int32_t num_seqs;             /* 1..DG_MAX_SEQS */
  const dg_kv_seq* seqs;        /* host array [num_seqs] */
  int32_t num_kv_heads;         /* Hkv >= 1 */
  int32_t head_dim;             /* D >= 8, a multiple of 8 */
  int32_t dtype;                /* dg_dtype of k_new and v_new (and of the pools unless pool_fp8) */
  int32_t block_size;           /* a power of two >= 1 */
  const int32_t* block_table;   /* device [block_table_len] int32 */
  int64_t block_table_len;      /* every request needs table_start + ceil((pos + num) / block_size) <= this */
  int64_t total_new;            /* rows of k_new / v_new */
  int64_t pool_rows;            /* rows of k_pool / v_pool, a multiple of block_size */
  const void* k_new;            /* device [total_new, Hkv, D] */
  const void* v_new;            /* device [total_new, Hkv, D] */
  void* k_pool;                 /* device [pool_rows, Hkv, D], dtype, or E4M3 codes when pool_fp8 */
  void* v_pool;                 /* device [pool_rows, Hkv, D], dtype, or E4M3 codes when pool_fp8 */
  int32_t pool_fp8;             /* 0: pools in dtype (a copy); 1: E4M3 pools, values quantized; other values
                                   and bad scales: DG_ERR_INVALID_ARG */
  float k_scale;                /* pool_fp8: finite, > 0; ignored otherwise */
  float v_scale;                /* pool_fp8: finite, > 0; ignored otherwise */
} dg_kv_write_args;

dg_status dg_kv_write(const dg_kv_write_args* args, void* stream);

/* ------------------------------------------------------------------------------
 * dg_selfcond_inject: the canvas embedding with the self-conditioning vector injected
 * ([P1] section "안정성을 위한 셀프 컨디셔닝": the probability-weighted average of token
 * embeddings is added to the canvas embedding through a gated MLP; section
 * "ModelState 인터페이스": prepare_inputs handles the canvas embedding and the
 * self-conditioning). The pages name the gated MLP but not its form; this call takes
 * the plainest one, a GeGLU with the tanh GELU, no bias:
 *   out[i, :] = embed[tokens[i], :] + (gelu(s[i] . Wg) * (s[i] . Wu)) . Wd
 *   gelu(x)   = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))
 * where Wg = w_gate_up[:, 0:hidden] and Wu = w_gate_up[:, hidden:2 hidden] (weights are
 * [in, out], row-major: x . W). Products accumulate in fp32; the gate/up product and
 * the GeGLU output are rounded to the input dtype, as is out.
 * ------------------------------------------------------------------------------ */
typedef struct {
  int32_t M;                    /* canvas rows, >= 1 */
  int32_t d;                    /* model width, a multiple of 128 */
  int32_t hidden;               /* MLP width, a multiple of 128 */
  int32_t vocab;                /* rows of embed, >= 1 */
  int32_t dtype;                /* dg_dtype of every float tensor */
  const int32_t* tokens;        /* device [M] canvas tokens; an entry outside [0, vocab) is clamped into it */
  const void* embed;            /* device [vocab, d] token embedding table */
  const void* s;                /* device [M, d] self-conditioning vectors (dg_selfcond_embed's output) */
  const void* w_gate_up;        /* device [d, 2 * hidden] */
  const void* w_down;           /* device [hidden, d] */
  void* out;                    /* device [M, d] */
  void* workspace;              /* device, >= dg_selfcond_inject_workspace_size(args) bytes */
  size_t workspace_bytes;
} dg_inject_args;

dg_status dg_selfcond_inject(const dg_inject_args* args, void* stream);
size_t dg_selfcond_inject_workspace_size(const dg_inject_args* args);

/* ------------------------------------------------------------------------------ */
const char* dg_status_string(dg_status s); /* static string for a status */
const char* dg_last_error(void);           /* message of this thread's last failed call */
int dg_abi_version(void);                  /* DG_ABI_VERSION */

/* Test hook, not for production use. With on != 0, every later dg_attn_mixed call (from
 * any thread) plans all its requests on the register-staged attention kernel, the one
 * that otherwise serves head_dim 64/128, fp32, FP8 K/V at head_dim 64/128, and contiguous
 * head_dim-256 requests whose K/V span passes 2^31 - 1 bytes; results stay within the
 * same bars, not bit-equal to the LDS-DMA kernels. on = 0 restores the normal per-request choice.
 * Returns the previous setting (0 or 1). */
int dg_test_force_register_staged(int on);

/* Test hook, not for production use. A head_dim-256 request (bf16 or FP8 K/V) runs on a
 * 64-rows-per-wave attention kernel when its work groups would average at least this many
 * 32-key sub-tiles (default 64), else on a 128-row kernel; this sets the number for
 * every later dg_attn_mixed call (from any thread), so that tests reach the first kernel
 * at small shapes. n < 1 restores the default. Results stay within the same bars; each
 * request's kernel still depends on that request alone. Returns the previous number. */
int dg_test_wide_min_sub(int n);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
