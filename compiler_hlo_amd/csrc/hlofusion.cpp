// hlofusion.cpp -- the C ABI: create (intake, plan, generate, compile, load),
// launch, destroy, and the hiprtc compile cache.
#include "hlofusion.h"

#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>
#include <unistd.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <memory>
#include <atomic>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "ir.h"
#include "plan.h"
#include "scratch.h"

// Device templates, embedded at build time: k_src_common, k_src_loop,
// k_src_transpose, k_src_reduce_row, k_src_reduce_col.
#include "kernels_embed.inc"

struct hf_fusion {
  hf::Graph g;
  hf::Plan P;
  std::string source;
  std::vector<char> code;
  bool plan_only = false, compile_only = false;
  int device = -1;
  hipModule_t mod = nullptr;
  hipFunction_t fn = nullptr;
  hipFunction_t fold = nullptr;  // column reduce: segment fold kernel
  std::vector<void *> qdev;  // scales, zero points per per-axis quant type
};

namespace {

thread_local std::string t_err;

void set_err(const std::string &m) { t_err = m; }

hf_status hip_fail(hipError_t e, const char *what) {
  set_err(std::string(what) + ": " + hipGetErrorString(e));
  return HF_ERR_HIP;
}

const char *hero_text(hf_hero h) {
  switch (h) {
    case HF_HERO_LOOP: return k_src_loop;
    case HF_HERO_TRANSPOSE: return k_src_transpose;
    case HF_HERO_ROW_REDUCE: return k_src_reduce_row;
    case HF_HERO_COLUMN_REDUCE: return k_src_reduce_col;
  }
  return "";
}

uint64_t fnv1a(const std::string &s, uint64_t h = 1469598103934665603ull) {
  for (unsigned char c : s) {
    h ^= c;
    h *= 1099511628211ull;
  }
  return h;
}

// Compile flags: gfx950, -O3, no FMA contraction (every op rounds once, as
// the op semantics define), no fast-math, packed FP32 instructions disabled.
const std::vector<const char *> &rtc_options() {
  static const std::vector<const char *> o = {
      "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fno-slp-vectorize",
      "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};
  return o;
}

// Compiled code objects of this process, keyed by the full compile input
// (options, compiler version, source): no two sources can share an entry.
std::mutex g_cache_mu;
std::map<std::string, std::vector<char>> g_cache;

hf_status compile(const std::string &src, std::vector<char> *code) {
  std::string opts;
  for (const char *o : rtc_options()) opts += std::string(o) + " ";
  int ver_major = 0, ver_minor = 0;
  hiprtcVersion(&ver_major, &ver_minor);
  const std::string full = opts + std::to_string(ver_major) + "." + std::to_string(ver_minor) + "\n" + src;
  const uint64_t key = fnv1a(full);
  {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    auto it = g_cache.find(full);
    if (it != g_cache.end()) {
      *code = it->second;
      return HF_OK;
    }
  }
  char name[64];
  std::snprintf(name, sizeof name, "hf_%016llx", (unsigned long long)key);
  const char *cdir = std::getenv("HF_CACHE_DIR");
  std::string cpath = cdir && *cdir ? std::string(cdir) + "/" + name + ".co" : "";
  if (!cpath.empty()) {
    std::ifstream f(cpath, std::ios::binary);
    if (f) {
      code->assign(std::istreambuf_iterator<char>(f), std::istreambuf_iterator<char>());
      if (!code->empty()) {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        g_cache[full] = *code;
        return HF_OK;
      }
    }
  }
  hiprtcProgram prog;
  std::string fname = std::string(name) + ".hip";
  if (hiprtcCreateProgram(&prog, src.c_str(), fname.c_str(), 0, nullptr, nullptr) != HIPRTC_SUCCESS) {
    set_err("hiprtcCreateProgram failed");
    return HF_ERR_COMPILE;
  }
  hiprtcResult r = hiprtcCompileProgram(prog, (int)rtc_options().size(), rtc_options().data());
  if (r != HIPRTC_SUCCESS) {
    size_t n = 0;
    hiprtcGetProgramLogSize(prog, &n);
    std::string log(n, '\0');
    if (n) hiprtcGetProgramLog(prog, &log[0]);
    hiprtcDestroyProgram(&prog);
    set_err(std::string("kernel compile failed: ") + hiprtcGetErrorString(r) + "\n" + log.substr(0, 4000));
    return HF_ERR_COMPILE;
  }
  size_t sz = 0;
  if (hiprtcGetCodeSize(prog, &sz) != HIPRTC_SUCCESS || sz == 0) {
    hiprtcDestroyProgram(&prog);
    set_err("hiprtcGetCodeSize failed");
    return HF_ERR_COMPILE;
  }
  code->resize(sz);
  r = hiprtcGetCode(prog, code->data());
  hiprtcDestroyProgram(&prog);
  if (r != HIPRTC_SUCCESS) {
    set_err(std::string("hiprtcGetCode failed: ") + hiprtcGetErrorString(r));
    return HF_ERR_COMPILE;
  }
  if (!cpath.empty()) {
    // unique per process and call: threads of one process may compile the
    // same source at once
    static std::atomic<unsigned long> tmp_seq{0};
    std::string tmp = cpath + ".tmp" + std::to_string((long)getpid()) + "." + std::to_string(tmp_seq.fetch_add(1));
    std::ofstream f(tmp, std::ios::binary);
    f.write(code->data(), (std::streamsize)code->size());
    f.close();
    std::rename(tmp.c_str(), cpath.c_str());
  }
  std::lock_guard<std::mutex> lk(g_cache_mu);
  g_cache[full] = *code;
  return HF_OK;
}

std::string plan_text(const hf_fusion *f) {
  std::ostringstream s;
  const hf_plan_info &i = f->P.info;
  s << "hero " << hf::hero_template_name(i.hero) << "\npartitions " << i.n_partitions << "\nvector_elems "
    << i.vector_elems << "\nblock " << i.block_threads << "\ngrid " << i.grid_blocks << "\nlds_bytes " << i.lds_bytes
    << "\nworkspace_bytes " << i.workspace_bytes << "\nalgorithmic_bytes " << i.algorithmic_bytes << "\nelements "
    << i.elements << "\nrows " << i.rows << "\ncols " << i.cols << "\n";
  for (size_t c = 0; c < f->P.ctx.size(); ++c) {
    s << "context " << c << ": root " << f->P.ctx[c].root << " lane " << f->P.ctx[c].lane << " V " << f->P.ctx[c].V
      << " partitions";
    for (int r : f->P.ctx[c].part_root) s << " " << r;
    s << "\n";
  }
  return s.str();
}

void dump(const hf_fusion *f) {
  const char *d = std::getenv("HF_DUMP");
  if (!d || !*d) return;
  char name[64];
  std::snprintf(name, sizeof name, "hf_%016llx", (unsigned long long)fnv1a(f->source));
  std::ofstream(std::string(d) + "/" + name + ".hip") << f->source;
  std::ofstream(std::string(d) + "/" + name + ".plan.txt") << plan_text(f);
}

// Frees what create made.  The caller has made sure that no launch of the
// handle is still running (hf_fusion_destroy waits for the device first; a
// handle that failed inside create was never launched).
void release(hf_fusion *f) {
  if (!f) return;
  if (f->mod) (void)hipModuleUnload(f->mod);
  for (void *p : f->qdev)
    if (p) (void)hipFree(p);
  delete f;
}

hf_status load_on_device(hf_fusion *f) {
  hipError_t e = hipGetDevice(&f->device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, f->device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    set_err(std::string("this library targets gfx950 (MI355X); current device is ") + prop.gcnArchName);
    return HF_ERR_UNSUPPORTED;
  }
  {
    // set-up of the no-allocation launch: this device's scratch address
    std::string err;
    const hf_status st = hf::scratch_prepare(f->device, &err);
    if (st != HF_OK) {
      set_err(err);
      return st;
    }
  }
  e = hipModuleLoadData(&f->mod, f->code.data());
  if (e != hipSuccess) return hip_fail(e, "hipModuleLoadData");
  e = hipModuleGetFunction(&f->fn, f->mod, f->P.kernel_name.c_str());
  if (e != hipSuccess) return hip_fail(e, "hipModuleGetFunction");
  if (f->P.fold_grid > 0) {
    e = hipModuleGetFunction(&f->fold, f->mod, f->P.fold_name.c_str());
    if (e != hipSuccess) return hip_fail(e, "hipModuleGetFunction(fold)");
  }
  f->qdev.reserve(3 * f->P.quant_args.size());  // push_back below cannot throw
  for (int q : f->P.quant_args) {
    const hf::Quant &Q = f->g.quants[q];
    void *s = nullptr, *z = nullptr;
    size_t n = Q.scales.size();
    e = hipMalloc(&s, n * 4 + 16);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(scales)");
    f->qdev.push_back(s);
    e = hipMalloc(&z, n + 16);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(zero points)");
    f->qdev.push_back(z);
    void *rc = nullptr;
    e = hipMalloc(&rc, n * 8 + 16);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(reciprocal scales)");
    f->qdev.push_back(rc);
    std::vector<signed char> zb(n);
    for (size_t i = 0; i < n; ++i) zb[i] = (signed char)Q.zero_points[i];  // u8 keeps its bit pattern
    std::vector<double> rb(n);
    for (size_t i = 0; i < n; ++i) rb[i] = hf::reciprocal(Q.scales[i]);
    if ((e = hipMemcpy(s, Q.scales.data(), n * 4, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(scales)");
    if ((e = hipMemcpy(z, zb.data(), n, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(zero points)");
    if ((e = hipMemcpy(rc, rb.data(), n * 8, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(reciprocal scales)");
  }
  return HF_OK;
}

// The launch behind the entry points.  check_ws: the workspace is the
// caller's and is checked like the other buffers (the library's own scratch
// memory is not).
hf_status launch(hf_fusion *f, const void *const *params, int32_t n_params, void *result, void *workspace,
                 bool check_ws, void *stream) {
  if (!f) {
    set_err("NULL handle");
    return HF_ERR_INVALID;
  }
  if (f->plan_only || f->compile_only || !f->fn) {
    set_err("the handle was created without loading a kernel (plan-only or compile-only)");
    return HF_ERR_INVALID;
  }
  if (n_params != f->g.n_params || (n_params > 0 && !params)) {
    set_err("expected " + std::to_string(f->g.n_params) + " parameter pointers, got " + std::to_string(n_params));
    return HF_ERR_INVALID;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != f->device) {
    set_err("the current device differs from the device the fusion was created on");
    return HF_ERR_INVALID;
  }
  // A buffer must be device memory of this device (or managed memory), with
  // its whole extent inside one allocation: anything else is rejected here,
  // before a kernel could fault on it.
  auto check_buffer = [&](const void *p, size_t bytes, const std::string &what) -> bool {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
      (void)hipGetLastError();  // do not leave the failed query to the next call
      set_err(what + " is not device memory");
      return false;
    }
    const bool managed = a.isManaged || a.type == hipMemoryTypeManaged;
    if (!managed && (a.type != hipMemoryTypeDevice || a.device != f->device)) {
      set_err(what + " is not device memory of the fusion's device");
      return false;
    }
    if (!managed) {
      hipDeviceptr_t base = nullptr;
      size_t size = 0;
      if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess) {
        (void)hipGetLastError();
        set_err(what + ": hipMemGetAddressRange failed");
        return false;
      }
      if ((uintptr_t)p + bytes > (uintptr_t)base + size) {
        set_err(what + " extends past the end of its allocation");
        return false;
      }
    }
    return true;
  };
  const hf::Type &rt = f->g.nodes[f->g.root].t;
  const size_t rbytes = (size_t)hf::storage_bytes(rt.dt, rt.numel());
  const uintptr_t r0 = (uintptr_t)result;
  const uintptr_t r1 = r0 + (uintptr_t)rbytes;
  if (rt.numel() > 0 && (!result || (r0 & 15))) {
    set_err("result must be a non-NULL, 16-byte aligned device pointer");
    return HF_ERR_INVALID;
  }
  if (rt.numel() > 0 && !check_buffer(result, rbytes, "the result")) return HF_ERR_INVALID;
  for (int k = 0; k < n_params; ++k) {
    int pn = f->g.param_node[k];
    if (pn < 0) continue;
    const hf::Type &pt = f->g.nodes[pn].t;
    if (pt.numel() == 0) continue;
    uintptr_t p0 = (uintptr_t)params[k], p1 = p0 + (uintptr_t)hf::storage_bytes(pt.dt, pt.numel());
    if (!params[k] || (p0 & 15)) {
      set_err("parameter " + std::to_string(k) + " must be a non-NULL, 16-byte aligned device pointer");
      return HF_ERR_INVALID;
    }
    if (!check_buffer(params[k], (size_t)(p1 - p0), "parameter " + std::to_string(k))) return HF_ERR_INVALID;
    if (rt.numel() > 0 && p0 < r1 && r0 < p1) {
      set_err("the result buffer overlaps parameter " + std::to_string(k));
      return HF_ERR_INVALID;
    }
  }
  // The workspace: scratch for this launch only (a column reduce's segment
  // partials), in the caller's memory, so that launches in flight at the
  // same time never share it.
  const size_t wbytes = (size_t)f->P.ws_bytes;
  if (wbytes > 0 && check_ws) {
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + wbytes;
    if (!workspace || (w0 & 15)) {
      set_err("this fusion needs a workspace of " + std::to_string(wbytes) +
              " bytes: a non-NULL, 16-byte aligned device pointer");
      return HF_ERR_INVALID;
    }
    if (!check_buffer(workspace, wbytes, "the workspace")) return HF_ERR_INVALID;
    if (rt.numel() > 0 && w0 < r1 && r0 < w1) {
      set_err("the workspace overlaps the result buffer");
      return HF_ERR_INVALID;
    }
    for (int k = 0; k < n_params; ++k) {
      int pn = f->g.param_node[k];
      if (pn < 0) continue;
      const hf::Type &pt = f->g.nodes[pn].t;
      const uintptr_t p0 = (uintptr_t)params[k], p1 = p0 + (uintptr_t)hf::storage_bytes(pt.dt, pt.numel());
      if (pt.numel() > 0 && p0 < w1 && w0 < p1) {
        set_err("the workspace overlaps parameter " + std::to_string(k));
        return HF_ERR_INVALID;
      }
    }
  }
  if (f->P.empty) return HF_OK;
  // Kernel arguments, in the generated kernel's order: parameters, result,
  // the per-axis quantization arrays, the workspace.  On the stack: a launch
  // allocates nothing.
  constexpr int kMaxArgs = HF_MAX_NODES + 1 + 3 * HF_MAX_NODES + 1;
  void *vals[kMaxArgs];
  void *ptrs[kMaxArgs];
  int na = 0;
  for (int k = 0; k < n_params; ++k) vals[na++] = const_cast<void *>(params[k]);
  vals[na++] = result;
  for (void *q : f->qdev) vals[na++] = q;
  vals[na++] = wbytes > 0 ? workspace : nullptr;
  for (int k = 0; k < na; ++k) ptrs[k] = &vals[k];
  e = hipModuleLaunchKernel(f->fn, (unsigned)f->P.grid, 1, 1, (unsigned)f->P.block, 1, 1, 0, (hipStream_t)stream,
                            ptrs, nullptr);
  if (e != hipSuccess) return hip_fail(e, "hipModuleLaunchKernel");
  if (f->fold) {
    e = hipModuleLaunchKernel(f->fold, (unsigned)f->P.fold_grid, 1, 1, 256, 1, 1, 0, (hipStream_t)stream, ptrs,
                              nullptr);
    if (e != hipSuccess) return hip_fail(e, "hipModuleLaunchKernel(fold)");
  }
  return HF_OK;
}

}  // namespace

namespace hf {

hf_status launch_in_scratch(hf_fusion *f, const void *const *params, int32_t n_params, void *result, void *stream) {
  if (!f) {
    set_err("NULL handle");
    return HF_ERR_INVALID;
  }
  const long long need = f->P.ws_bytes;
  if (need > (long long)HF_SCRATCH_BYTES) {
    set_err("this fusion needs " + std::to_string(need) + " bytes of workspace, more than the " +
            std::to_string((long long)HF_SCRATCH_BYTES) +
            " bytes of the library's scratch memory: launch it with hf_fusion_launch and a workspace");
    return HF_ERR_UNSUPPORTED;
  }
  void *ws = nullptr;
  if (need > 0 && !(ws = scratch_address(f->device))) {
    set_err("no scratch memory was set up on the fusion's device (the handle was not loaded on a device)");
    return HF_ERR_INVALID;
  }
  return launch(f, params, n_params, result, ws, false, stream);
}

}  // namespace hf

extern "C" {

const char *hf_last_error(void) { return t_err.c_str(); }

int32_t hf_abi_version(void) { return HF_ABI_VERSION; }

int64_t hf_linear_index(int32_t rank, const int64_t *dims, const int32_t *m2m, const int64_t *index) {
  if (rank < 0 || rank > HF_MAX_RANK || (rank > 0 && (!dims || !m2m || !index))) return -1;
  // linear = sum over k of index[m2m[k]] * stride_k, stride_0 = 1,
  // stride_{k+1} = stride_k * dims[m2m[k]]  (Shapes and layout, "Array indexing")
  int64_t lin = 0, stride = 1;
  bool seen[HF_MAX_RANK] = {false};
  for (int k = 0; k < rank; ++k) {
    int d = m2m[k];
    if (d < 0 || d >= rank || seen[d] || index[d] < 0 || index[d] >= dims[d]) return -1;
    seen[d] = true;
    int64_t term;
    if (__builtin_mul_overflow(index[d], stride, &term) || __builtin_add_overflow(lin, term, &lin) ||
        __builtin_mul_overflow(stride, dims[d], &stride))
      return -1;
  }
  return lin;
}

hf_status hf_fusion_create(const hf_fusion_desc *desc, uint32_t flags, hf_fusion **out) {
  t_err.clear();
  if (!out) {
    set_err("out is NULL");
    return HF_ERR_INVALID;
  }
  *out = nullptr;
  // No exception crosses the C boundary.
  try {
    // The deleter frees whatever was loaded, on every early return and on
    // exceptions alike.
    std::unique_ptr<hf_fusion, void (*)(hf_fusion *)> f(new hf_fusion, release);
    f->g = hf::intake(desc);
    f->P = hf::make_plan(f->g);
    f->plan_only = flags & HF_CREATE_PLAN_ONLY;
    f->compile_only = flags & HF_CREATE_COMPILE_ONLY;
    if (!f->plan_only) {
      std::string prelude = k_src_common;
      // The source text names the compiler options too, so that anything
      // keyed on the text (measurements of a kernel) changes with them.
      std::string opts = "// hiprtc options:";
      for (const char *o : rtc_options()) opts += std::string(" ") + o;
      f->source = opts + "\n" + hf::generate_source(f->g, f->P, prelude, hero_text(f->P.hero));
      dump(f.get());
      hf_status st = compile(f->source, &f->code);
      if (st != HF_OK) return st;
      if (!f->compile_only) {
        st = load_on_device(f.get());
        if (st != HF_OK) return st;
      }
    }
    *out = f.release();
    return HF_OK;
  } catch (const hf::Error &e) {
    set_err(e.msg);
    return e.status;
  } catch (const std::bad_alloc &) {
    set_err("out of host memory");
    return HF_ERR_NOMEM;
  } catch (const std::exception &e) {
    set_err(std::string("internal error: ") + e.what());
    return HF_ERR_INVALID;
  } catch (...) {
    set_err("internal error");
    return HF_ERR_INVALID;
  }
}

hf_status hf_fusion_plan(const hf_fusion *f, hf_plan_info *info) {
  if (!f || !info) {
    set_err("NULL argument");
    return HF_ERR_INVALID;
  }
  *info = f->P.info;
  return HF_OK;
}

hf_status hf_fusion_source(const hf_fusion *f, char *buf, size_t cap, size_t *len) {
  if (!f) {
    set_err("NULL handle");
    return HF_ERR_INVALID;
  }
  if (f->plan_only) {
    set_err("the handle was created with HF_CREATE_PLAN_ONLY: no source");
    return HF_ERR_INVALID;
  }
  if (len) *len = f->source.size();
  if (buf && cap > f->source.size()) std::memcpy(buf, f->source.c_str(), f->source.size() + 1);
  return HF_OK;
}

hf_status hf_fusion_launch(hf_fusion *f, const void *const *params, int32_t n_params, void *result, void *workspace,
                           void *stream) {
  return launch(f, params, n_params, result, workspace, true, stream);
}

hf_status hf_fusion_destroy(hf_fusion *f) {
  if (!f) return HF_OK;
  if (f->mod) {
    // Launches of the handle may still be running: wait for the device
    // before the code object and the quantization arrays go away.
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != f->device && (e = hipSetDevice(f->device)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    e = hipDeviceSynchronize();
    if (cur != f->device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize before releasing the fusion (nothing released)");
  }
  release(f);
  return HF_OK;
}

}  // extern "C"
