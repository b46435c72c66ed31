// Runtime shape specialisation of the GEMM kernels (declared in fp8gemm.h).
//
// What it does ("DeepSeek open-source week, day 3: DeepGEMM", "Core
// features": kernels compiled at run time per shape and cached; its
// environment-variable list: a cache directory and JIT debug output; the
// kwkr.cn usage article, sections 2.3 and 3.3: per-shape compilation, a
// warm-up before timing, and a cache that survives restarts):
//   * gemm_kernel<...> is instantiated for a tile configuration (tile size,
//     wave grid, ring depth, K groups per stage, split-K) and, on request,
//     with n and k as compile-time constants, and compiled for the device's
//     own target by the ROCm compiler run as a child process (as the pages'
//     JIT runs its compiler), with the device code-generation options of the
//     ahead-of-time build, so the code equals the ahead-of-time code for the
//     same configuration.  A child process rather than hipRTC: in a process
//     that has loaded another ROCm runtime (a framework's bundled copy), the
//     in-process compiler is that runtime's, with its own option set, and an
//     option it does not know ends the process;
//   * code objects are kept in an on-disk cache keyed by everything that
//     determines them (kernel source digest, target, options, the
//     instantiation), written atomically and checked on load (a damaged or
//     foreign file is counted, ignored and replaced);
//   * loaded kernels are kept per device for the life of the process.
// The launch path is the ahead-of-time one: same parameter block, grid and
// workspace layout.
#include <hip/hip_runtime.h>

#include <fcntl.h>
#include <spawn.h>
#include <sys/stat.h>
#include <sys/wait.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cerrno>
#include <cstring>
#include <fstream>
#include <mutex>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "fp8gemm.h"
#include "gemm_kernel.hpp"
#include "host_common.hpp"
#include "jit_sources.inc"

extern char** environ;

namespace {

using fp8g::GemmParams;
using namespace fp8g::host;

constexpr char kMagic[8] = {'F', 'P', '8', 'G', 'J', 'I', 'T', '1'};

std::atomic<long long> g_stat[5];  // memory hits, disk hits, compiles, rejected files, failed compiles
enum { kMemHit, kDiskHit, kCompile, kRejected, kFailed };

bool jit_debug() {
  static const bool on = [] {
    const char* v = std::getenv("FP8G_JIT_DEBUG");
    return v && v[0] == '1';
  }();
  return on;
}

uint64_t fnv1a(const void* data, size_t len, uint64_t h = 1469598103934665603ull) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < len; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

uint64_t source_digest() {
  static const uint64_t d = [] {
    uint64_t h = 1469598103934665603ull;
    for (int i = 0; i < fp8g::jit_src::kNumHeaders; ++i) {
      h = fnv1a(fp8g::jit_src::kHeaderNames[i], std::strlen(fp8g::jit_src::kHeaderNames[i]), h);
      h = fnv1a(fp8g::jit_src::kHeaderTexts[i], std::strlen(fp8g::jit_src::kHeaderTexts[i]), h);
    }
    return h;
  }();
  return d;
}

std::mutex g_mu;                          // guards the tables below
std::condition_variable g_built;          // a kernel left g_building
std::unordered_set<std::string> g_building;  // kernels being read, compiled or loaded
std::string g_cache_dir;                  // empty: not chosen yet

std::string compiler_path() {
  if (const char* c = std::getenv("FP8G_JIT_COMPILER"); c && *c) return c;
  if (const char* r = std::getenv("ROCM_PATH"); r && *r) return std::string(r) + "/llvm/bin/clang++";
  return "/opt/rocm/llvm/bin/clang++";
}

std::string default_cache_dir() {
  if (const char* d = std::getenv("FP8G_CACHE_DIR"); d && *d) return d;
  if (const char* h = std::getenv("HOME"); h && *h) return std::string(h) + "/.cache/fp8gemm";
  return "/tmp/fp8gemm-cache";
}

const std::string& cache_dir_locked() {
  if (g_cache_dir.empty()) g_cache_dir = default_cache_dir();
  return g_cache_dir;
}

bool make_dirs(const std::string& path) {
  if (path.empty()) return false;
  std::string cur;
  size_t pos = 0;
  while (pos != std::string::npos) {
    pos = path.find('/', pos + 1);
    cur = path.substr(0, pos);
    if (cur.empty()) continue;
    if (mkdir(cur.c_str(), 0755) != 0 && errno != EEXIST) return false;
  }
  return true;
}

// Target of the current device ("gfx950:sramecc+:xnack-").  With no device
// (compile-only use: filling a disk cache, e.g. for another machine) it is
// $FP8G_JIT_TARGET, else gfx950.
std::string device_arch(int* device) {
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.gcnArchName[0]) {
      *device = dev;
      return prop.gcnArchName;
    }
  }
  (void)hipGetLastError();
  *device = -1;
  if (const char* t = std::getenv("FP8G_JIT_TARGET"); t && *t) return t;
  return "gfx950";
}

struct Program {
  std::string expr;      // template instantiation
  std::string symbol;    // its mangled kernel name
  int threads = 0;       // workgroup size
};

struct Loaded {
  hipModule_t module = nullptr;
  hipFunction_t fn = nullptr;
};
std::unordered_map<std::string, Loaded> g_loaded;  // "<device>|<key>" -> kernel
std::unordered_set<std::string> g_refused;                  // "<device>|<key>" of refused builds

// ---- configurations ------------------------------------------------------
bool valid_config(const fp8_gemm_config& c, int mode) {
  const int nw = c.waves_m * c.waves_n * c.waves_k;
  if (c.waves_m < 1 || c.waves_n < 1 || c.waves_k < 1 || (nw != 4 && nw != 8)) return false;
  if (c.block_m < 16 || c.block_m > 256 || c.block_n < 16 || c.block_n > 256) return false;
  if (c.block_m % c.waves_m || c.block_n % c.waves_n) return false;
  const int wm = c.block_m / c.waves_m, wn = c.block_n / c.waves_n;
  if (wm % 16 || wn % 16 || wn > 128 || 128 % wn) return false;
  if (c.block_m % (8 * nw) || c.block_n % (8 * nw)) return false;
  if (c.stages < 1 || c.stages > 8 || c.k_per_stage < 1 || c.k_per_stage > 4 || c.k_per_stage % c.waves_k)
    return false;
  const int copies = c.k_per_stage * (c.block_m / (8 * nw) + c.block_n / (8 * nw));
  if ((c.stages - 2) * copies >= 64) return false;  // vmcnt range
  const int slots = c.stages * c.k_per_stage;
  const int ring = slots * (c.block_m * 128 + c.block_n * 128 + c.block_m * 4);
  const int sb_blocks = (c.block_n + 127) / 128;
  const int staging = c.block_m * (c.block_n + 8) * 2;  // the BF16 output tile on its way out
  const int partial = c.splits > 1 ? c.block_m * (c.block_n + 4) * 4 : 0;  // a split's FP32 tile
  if (std::max(std::max(ring, staging), partial) + sb_blocks * fp8g::kMaxGroups * 4 > 160 * 1024)
    return false;  // LDS
  const int tm = wm / 16, tn = wn / 16;
  if (tm * tn > 32) return false;  // accumulators stay within 128 VGPRs
  if (c.waves_k > 1 && nw * tn * tm * 64 * 16 > ring) return false;
  if (c.splits < 1 || c.splits > fp8g::kMaxSplits) return false;
  if (c.splits > 1 && mode != FP8G_JIT_DENSE) return false;
  if (mode == FP8G_JIT_CONTIGUOUS && c.block_m != 256) return false;
  return mode == FP8G_JIT_DENSE || mode == FP8G_JIT_CONTIGUOUS || mode == FP8G_JIT_MASKED;
}

fp8_gemm_config from_shape(const KernelShape& ks, int splits) {
  fp8_gemm_config c{};
  c.block_m = ks.bm; c.block_n = ks.bn;
  c.waves_m = ks.wm; c.waves_n = ks.wn; c.waves_k = ks.wk;
  c.stages = ks.stages; c.k_per_stage = ks.ku; c.splits = splits; c.specialize = 0;
  return c;
}

Program program_for(const fp8_gemm_config& c, int mode, int fmt, int n, int k) {
  const int nspec = c.specialize ? n : 0, kspec = c.specialize ? k : 0;
  const bool split = c.splits > 1;
  char buf[256];
  std::snprintf(buf, sizeof(buf), "fp8g::gemm_kernel<%d, %d, %d, %d, %d, %d, %s, %d, %d, %d, %d, %d>", c.block_m,
                c.block_n, c.waves_m, c.waves_n, c.stages, mode, split ? "true" : "false", c.k_per_stage,
                c.waves_k, fmt, nspec, kspec);
  Program p;
  p.expr = buf;
  // Itanium mangling of fp8g::gemm_kernel<ints..., bool, ints...>(fp8g::GemmParams)
  auto lit = [](int v) { return "Li" + (v < 0 ? "n" + std::to_string(-v) : std::to_string(v)) + "E"; };
  p.symbol = "_ZN4fp8g11gemm_kernelI" + lit(c.block_m) + lit(c.block_n) + lit(c.waves_m) + lit(c.waves_n) +
             lit(c.stages) + lit(mode) + (split ? "Lb1E" : "Lb0E") + lit(c.k_per_stage) + lit(c.waves_k) +
             lit(fmt) + lit(nspec) + lit(kspec) + "EEvNS_10GemmParamsE";
  p.threads = 64 * c.waves_m * c.waves_n * c.waves_k;
  return p;
}

std::string cache_key(const std::string& arch, const Program& prog) {
  char digest[32];
  std::snprintf(digest, sizeof(digest), "%016llx", (unsigned long long)source_digest());
  std::string key = "fp8gemm-jit-v1\n";
  key += arch + "\n";
  const std::string cc = compiler_path();
  struct stat st {};
  char ccid[64] = "";
  if (stat(cc.c_str(), &st) == 0)
    std::snprintf(ccid, sizeof(ccid), " %lld %lld", (long long)st.st_size, (long long)st.st_mtime);
  key += cc + ccid + "\n";
  for (int i = 0; i < fp8g::jit_src::kNumOptions; ++i) key += std::string(fp8g::jit_src::kOptions[i]) + " ";
  key += "\n" + prog.expr + "\n" + digest + "\n";
  return key;
}

std::string cache_file(const std::string& dir, const std::string& key) {
  char name[32];
  std::snprintf(name, sizeof(name), "%016llx.co", (unsigned long long)fnv1a(key.data(), key.size()));
  return dir + "/" + name;
}

// ---- disk cache ----------------------------------------------------------
// File: magic[8], u32 key length, u32 kernel-name length, u64 code length,
// u64 FNV-1a of the code, key, kernel name, code object.
struct Header {
  char magic[8];
  uint32_t key_len, name_len;
  uint64_t code_len, code_hash;
};

bool read_cached(const std::string& path, const std::string& key, std::string* name, std::vector<char>* code,
                 bool* rejected) {
  *rejected = false;
  std::ifstream f(path, std::ios::binary);
  if (!f) return false;
  f.seekg(0, std::ios::end);
  const std::streamoff size = f.tellg();
  f.seekg(0);
  Header h{};
  auto reject = [&](const char* why) {
    *rejected = true;
    if (jit_debug()) std::fprintf(stderr, "[fp8gemm jit] ignoring cache file %s: %s\n", path.c_str(), why);
    return false;
  };
  if (size < std::streamoff(sizeof(Header)) || !f.read(reinterpret_cast<char*>(&h), sizeof(h)))
    return reject("truncated header");
  if (std::memcmp(h.magic, kMagic, sizeof(kMagic)) != 0) return reject("bad magic");
  if (h.key_len != key.size() || h.name_len == 0 || h.name_len > 4096 ||
      uint64_t(size) != sizeof(Header) + h.key_len + h.name_len + h.code_len)
    return reject("inconsistent sizes");
  std::string k(h.key_len, '\0');
  name->assign(h.name_len, '\0');
  code->resize(h.code_len);
  if (!f.read(&k[0], h.key_len) || !f.read(&(*name)[0], h.name_len) || !f.read(code->data(), h.code_len))
    return reject("short read");
  if (k != key) return reject("key mismatch");
  if (fnv1a(code->data(), code->size()) != h.code_hash) return reject("checksum mismatch");
  return true;
}

void write_cached(const std::string& dir, const std::string& path, const std::string& key, const std::string& name,
                  const std::vector<char>& code) {
  if (!make_dirs(dir)) {
    if (jit_debug()) std::fprintf(stderr, "[fp8gemm jit] cache directory %s is not writable\n", dir.c_str());
    return;
  }
  static std::atomic<unsigned> seq{0};
  const std::string tmp = path + ".tmp" + std::to_string(getpid()) + "_" + std::to_string(seq.fetch_add(1));
  {
    std::ofstream f(tmp, std::ios::binary | std::ios::trunc);
    if (!f) return;
    Header h{};
    std::memcpy(h.magic, kMagic, sizeof(kMagic));
    h.key_len = uint32_t(key.size());
    h.name_len = uint32_t(name.size());
    h.code_len = code.size();
    h.code_hash = fnv1a(code.data(), code.size());
    f.write(reinterpret_cast<const char*>(&h), sizeof(h));
    f.write(key.data(), key.size());
    f.write(name.data(), name.size());
    f.write(code.data(), code.size());
    if (!f) {
      f.close();
      std::remove(tmp.c_str());
      return;
    }
  }
  if (std::rename(tmp.c_str(), path.c_str()) != 0) std::remove(tmp.c_str());
}

// ---- compilation -----------------------------------------------------------
bool write_file(const std::string& path, const char* data, size_t len) {
  static std::atomic<unsigned> seq{0};
  const std::string tmp = path + ".tmp" + std::to_string(getpid()) + "_" + std::to_string(seq.fetch_add(1));
  {
    std::ofstream f(tmp, std::ios::binary | std::ios::trunc);
    if (!f || !f.write(data, len)) {
      std::remove(tmp.c_str());
      return false;
    }
  }
  if (std::rename(tmp.c_str(), path.c_str()) != 0) {
    std::remove(tmp.c_str());
    return false;
  }
  return true;
}

// Runs argv[0] as a child process with stdout and stderr into `log`;
// returns its exit status (-1 if it could not run or did not exit).
int run_child(const std::vector<std::string>& argv, const std::string& log) {
  posix_spawn_file_actions_t fa;
  posix_spawn_file_actions_init(&fa);
  posix_spawn_file_actions_addopen(&fa, 0, "/dev/null", O_RDONLY, 0);
  posix_spawn_file_actions_addopen(&fa, 1, log.c_str(), O_WRONLY | O_CREAT | O_TRUNC, 0644);
  posix_spawn_file_actions_adddup2(&fa, 1, 2);
  std::vector<char*> args;
  for (const std::string& a : argv) args.push_back(const_cast<char*>(a.c_str()));
  args.push_back(nullptr);
  pid_t pid = -1;
  const int rc = posix_spawn(&pid, argv[0].c_str(), &fa, nullptr, args.data(), environ);
  posix_spawn_file_actions_destroy(&fa);
  if (rc != 0) return -1;
  int status = 0;
  while (waitpid(pid, &status, 0) < 0)
    if (errno != EINTR) return -1;
  return WIFEXITED(status) ? WEXITSTATUS(status) : -1;
}

std::string read_text(const std::string& path, size_t max_len) {
  std::ifstream f(path);
  std::string s((std::istreambuf_iterator<char>(f)), std::istreambuf_iterator<char>());
  return s.substr(0, max_len);
}

// Scratch bytes per lane the kernel in a code object needs: the value of
// ".private_segment_fixed_size" in its metadata note (a MessagePack map, so
// the key's bytes are followed by an unsigned integer); -1 if not found.
long long private_segment_size(const std::vector<char>& code) {
  static const char kKey[] = ".private_segment_fixed_size";
  const size_t klen = sizeof(kKey) - 1;
  long long worst = -1;
  for (size_t i = 0; i + klen + 9 <= code.size(); ++i) {
    if (std::memcmp(&code[i], kKey, klen) != 0) continue;
    const unsigned char* v = reinterpret_cast<const unsigned char*>(&code[i + klen]);
    long long val = -1;
    if (v[0] < 0x80) val = v[0];
    else if (v[0] == 0xcc) val = v[1];
    else if (v[0] == 0xcd) val = (v[1] << 8) | v[2];
    else if (v[0] == 0xce) val = (static_cast<long long>(v[1]) << 24) | (v[2] << 16) | (v[3] << 8) | v[4];
    worst = std::max(worst, val);
  }
  return worst;
}

// Name stored in a cache entry for a configuration whose build was refused
// (it needs scratch memory): later processes skip the doomed compilation.
const char kRefusedName[] = "!refused: needs scratch memory";

int compile(const std::string& dir, const std::string& arch, const std::string& key, const Program& prog,
            std::vector<char>* code, bool* refused) {
  *refused = false;
  const auto t0 = std::chrono::steady_clock::now();
  // the embedded headers, once per kernel-source digest
  char sub[48];
  std::snprintf(sub, sizeof(sub), "/src-%016llx", (unsigned long long)source_digest());
  const std::string src_dir = dir + sub, work = dir + "/tmp";
  if (!make_dirs(src_dir) || !make_dirs(work)) return FP8G_ELAUNCH;
  for (int i = 0; i < fp8g::jit_src::kNumHeaders; ++i) {
    const std::string h = src_dir + "/" + fp8g::jit_src::kHeaderNames[i];
    struct stat st {};
    const size_t len = std::strlen(fp8g::jit_src::kHeaderTexts[i]);
    if (stat(h.c_str(), &st) != 0 || size_t(st.st_size) != len)
      if (!write_file(h, fp8g::jit_src::kHeaderTexts[i], len)) return FP8G_ELAUNCH;
  }
  static std::atomic<unsigned> seq{0};
  char stem[96];
  std::snprintf(stem, sizeof(stem), "/k%016llx_%d_%u", (unsigned long long)fnv1a(key.data(), key.size()),
                int(getpid()), seq.fetch_add(1));
  const std::string src = work + stem + ".hip", obj = work + stem + ".co", log = work + stem + ".log";
  const std::string text = "#include \"gemm_kernel.hpp\"\ntemplate __global__ void " + prog.expr +
                           "(fp8g::GemmParams);\n";
  if (!write_file(src, text.data(), text.size())) return FP8G_ELAUNCH;
  std::vector<std::string> argv{compiler_path(), "-x", "hip", "--offload-arch=" + arch, "--cuda-device-only",
                                "--no-gpu-bundle-output"};
  for (int i = 0; i < fp8g::jit_src::kNumOptions; ++i) argv.push_back(fp8g::jit_src::kOptions[i]);
  // a fixed compilation-unit id (hip-clang derives one from the source path
  // otherwise), so a configuration always builds to the same bytes
  char cuid[40];
  std::snprintf(cuid, sizeof(cuid), "-cuid=%016llx", (unsigned long long)fnv1a(key.data(), key.size()));
  argv.insert(argv.end(), {cuid, "-I", src_dir, src, "-o", obj});
  const int rc = run_child(argv, log);
  std::ifstream f(obj, std::ios::binary);
  if (rc == 0 && f) code->assign(std::istreambuf_iterator<char>(f), std::istreambuf_iterator<char>());
  const bool ok = rc == 0 && code->size() > 4 && std::memcmp(code->data(), "\x7f" "ELF", 4) == 0;
  if (!ok && (jit_debug() || log_enabled()))
    std::fprintf(stderr, "[fp8gemm jit] compiling %s failed (status %d):\n%s\n", prog.expr.c_str(), rc,
                 read_text(log, 8000).c_str());
  std::remove(src.c_str());
  std::remove(obj.c_str());
  std::remove(log.c_str());
  if (!ok) {
    g_stat[kFailed]++;
    return rc == -1 ? FP8G_ELAUNCH : FP8G_EUNSUPPORTED;
  }
  // A build that spills registers to scratch is refused: it is slow, and
  // its spill traffic shares the vector-memory counter with the operand
  // copies that the ring waits count.
  if (private_segment_size(*code) != 0) {
    g_stat[kFailed]++;
    *refused = true;
    if (jit_debug() || log_enabled())
      std::fprintf(stderr, "[fp8gemm jit] %s needs scratch memory (register spills): refused\n",
                   prog.expr.c_str());
    return FP8G_EUNSUPPORTED;
  }
  g_stat[kCompile]++;
  if (jit_debug())
    std::fprintf(stderr, "[fp8gemm jit] compiled %s for %s in %.2f s\n", prog.expr.c_str(), arch.c_str(),
                 std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count());
  return FP8G_OK;
}

// The kernel for `prog` on the current device: from memory, else from the
// disk cache, else compiled (and written to the cache).  With no device the
// code object is only made available on disk and *fn stays null.  The lock
// covers only the tables: a compilation runs unlocked, so other kernels stay
// usable meanwhile, and a second caller of the same kernel waits for the
// first instead of compiling it again.
int get_kernel(const Program& prog, hipFunction_t* fn) {
  *fn = nullptr;
  int device = -1;
  const std::string arch = device_arch(&device);
  const std::string key = cache_key(arch, prog);
  const std::string mem_key = std::to_string(device) + "|" + key;
  std::string dir;
  {
    std::unique_lock<std::mutex> lock(g_mu);
    g_built.wait(lock, [&] { return g_building.count(mem_key) == 0; });
    if (g_refused.count(mem_key)) {
      g_stat[kMemHit]++;
      return FP8G_EUNSUPPORTED;
    }
    if (device >= 0) {
      auto it = g_loaded.find(mem_key);
      if (it != g_loaded.end()) {
        g_stat[kMemHit]++;
        *fn = it->second.fn;
        return FP8G_OK;
      }
    }
    g_building.insert(mem_key);
    dir = cache_dir_locked();
  }
  Loaded l;
  bool refused_here = false;
  const int st = [&] {
    const std::string path = cache_file(dir, key);
    std::string name;
    std::vector<char> code;
    bool rejected = false, refused = false;
    const bool cached = read_cached(path, key, &name, &code, &rejected);
    if (cached && name == kRefusedName) {
      g_stat[kDiskHit]++;
      if (jit_debug()) std::fprintf(stderr, "[fp8gemm jit] %s refused (recorded in %s)\n", prog.expr.c_str(),
                                    path.c_str());
      refused_here = true;
      return int(FP8G_EUNSUPPORTED);
    }
    if (cached && name == prog.symbol) {
      g_stat[kDiskHit]++;
      if (jit_debug()) std::fprintf(stderr, "[fp8gemm jit] %s from %s\n", prog.expr.c_str(), path.c_str());
    } else {
      if (rejected) g_stat[kRejected]++;
      if (const int c = compile(dir, arch, key, prog, &code, &refused)) {
        if (refused) {  // remembered on disk: later processes do not rebuild it
          write_cached(dir, path, key, kRefusedName, std::vector<char>());
          refused_here = true;
        }
        return c;
      }
      name = prog.symbol;
      write_cached(dir, path, key, name, code);
    }
    if (device < 0) return int(FP8G_OK);
    if (hipModuleLoadData(&l.module, code.data()) != hipSuccess ||
        hipModuleGetFunction(&l.fn, l.module, name.c_str()) != hipSuccess) {
      (void)hipGetLastError();
      return int(FP8G_ELAUNCH);
    }
    return int(FP8G_OK);
  }();
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (st == FP8G_OK && l.fn) g_loaded[mem_key] = l;  // kept until the process ends
    if (refused_here) g_refused.insert(mem_key);
    g_building.erase(mem_key);
  }
  g_built.notify_all();
  *fn = l.fn;
  return st;
}

int launch(const Program& prog, const GemmParams& p, int64_t grid, void* stream) {
  if (grid <= 0 || grid > 0x7fffffff) return FP8G_EUNSUPPORTED;
  hipFunction_t fn = nullptr;
  if (const int st = get_kernel(prog, &fn)) return st;
  if (!fn) return FP8G_ELAUNCH;  // no device
  GemmParams local = p;
  return launch_units(local, grid, [&](int64_t g) {
    void* args[] = {&local};
    if (hipModuleLaunchKernel(fn, unsigned(g), 1, 1, unsigned(prog.threads), 1, 1, 0,
                              static_cast<hipStream_t>(stream), args, nullptr) != hipSuccess) {
      (void)hipGetLastError();
      return int(FP8G_ELAUNCH);
    }
    return launched("jit gemm");
  });
}

// FP8G_PIPELINE_DEPTH=d (debugging): every runtime-specialised kernel is
// built with a ring of d stages, d = 1 being the single-buffer form in which
// no copy overlaps the products (a pipeline race then disappears, an
// arithmetic error does not).
void apply_debug_depth(fp8_gemm_config& c) {
  const int d = env_int("FP8G_PIPELINE_DEPTH", 0);
  if (d > 0) c.stages = d;
}

int format_code(int lhs_format, int rhs_format, int* fmt) {
  if ((lhs_format != FP8G_E4M3 && lhs_format != FP8G_E5M2) || (rhs_format != FP8G_E4M3 && rhs_format != FP8G_E5M2))
    return FP8G_EINVAL;
  *fmt = (lhs_format == FP8G_E5M2 ? 1 : 0) | (rhs_format == FP8G_E5M2 ? 2 : 0);
  return FP8G_OK;
}

// Dense tiling for a configuration: the split count is clamped to the K
// groups and rounded like the ahead-of-time path.
DenseConfig dense_tiling(const fp8_gemm_config& c, int m, int n, int k) {
  DenseConfig d{};
  d.kind = -1;
  d.tiles_m = int(cdiv(m, c.block_m));
  d.tiles_n = int(cdiv(n, c.block_n));
  const int kg = k / 128;
  const int s = std::max(1, std::min(c.splits, kg));
  d.gps = int(cdiv(kg, s));
  d.splits = int(cdiv(kg, d.gps));
  return d;
}

}  // namespace

extern "C" {

int fp8_jit_default_config(int mode, int m, int n, int k, fp8_gemm_config* config) {
  if (!config || m < 0) return FP8G_EINVAL;
  if (const int st = check_gemm_shape(n, k)) return st;
  if (mode == FP8G_JIT_DENSE) {
    const DenseConfig d = dense_config(std::max(m, 1), std::max(n, 8), k, true);
    *config = from_shape(kShapes[d.kind], d.splits);
  } else if (mode == FP8G_JIT_CONTIGUOUS) {
    *config = from_shape(kContiguousShape, 1);
  } else if (mode == FP8G_JIT_MASKED) {
    *config = from_shape(kMaskedShape, 1);
  } else {
    return FP8G_EINVAL;
  }
  return FP8G_OK;
}

int fp8_jit_config_supported(int mode, const fp8_gemm_config* config) {
  if (!config) return FP8G_EINVAL;
  return valid_config(*config, mode) ? FP8G_OK : FP8G_EUNSUPPORTED;
}

int fp8_jit_warmup(int mode, int n, int k, int lhs_format, int rhs_format, const fp8_gemm_config* config) {
  int fmt = 0;
  if (const int st = format_code(lhs_format, rhs_format, &fmt)) return st;
  if (const int st = check_gemm_shape(n, k)) return st;
  fp8_gemm_config c{};
  if (config) c = *config;
  else if (const int st = fp8_jit_default_config(mode, 1, n, k, &c)) return st;
  apply_debug_depth(c);
  if (!valid_config(c, mode)) return FP8G_EUNSUPPORTED;
  hipFunction_t fn = nullptr;
  return get_kernel(program_for(c, mode, fmt, n, k), &fn);
}

size_t fp8_jit_gemm_workspace_bytes(int m, int n, int k, const fp8_gemm_config* config) {
  if (!config || m <= 0 || n <= 0 || k <= 0 || k % 128 != 0 || !valid_config(*config, FP8G_JIT_DENSE)) return 0;
  return dense_workspace(dense_tiling(*config, m, n, k), m, n);
}

int fp8_jit_gemm_nt(const uint8_t* lhs, int lhs_format, const float* lhs_scales, int64_t lhs_scales_ld,
                    const uint8_t* rhs, int rhs_format, const float* rhs_scales, uint16_t* out, int m, int n, int k,
                    const fp8_gemm_config* config, void* workspace, size_t workspace_bytes, void* stream) {
  int fmt = 0;
  if (m < 0) return FP8G_EINVAL;
  if (const int st = format_code(lhs_format, rhs_format, &fmt)) return st;
  if (const int st = check_gemm_shape(n, k)) return st;
  if (m == 0 || n == 0) return FP8G_OK;
  if (!lhs || !lhs_scales || !rhs || !rhs_scales || !out) return FP8G_EINVAL;
  if (!aligned16(lhs) || !aligned16(lhs_scales) || !aligned16(rhs) || !aligned16(rhs_scales) || !aligned16(out) ||
      (workspace && !aligned16(workspace)))
    return FP8G_EINVAL;
  if (const int st = check_ld(lhs_scales_ld, m)) return st;
  fp8_gemm_config c{};
  if (config) c = *config;
  else fp8_jit_default_config(FP8G_JIT_DENSE, m, n, k, &c);
  apply_debug_depth(c);
  if (!valid_config(c, FP8G_JIT_DENSE)) return FP8G_EUNSUPPORTED;
  DenseConfig d = dense_tiling(c, m, n, k);
  if (d.splits > 1 && (!workspace || workspace_bytes < dense_workspace(d, m, n))) {
    c.splits = 1;  // as the ahead-of-time path: too little workspace means no split
    d = dense_tiling(c, m, n, k);
  }
  c.splits = d.splits;

  GemmParams p{};
  p.a = lhs; p.sa = lhs_scales; p.b = rhs; p.sb = rhs_scales; p.out = out;
  if (d.splits > 1) {
    p.tile_counters = static_cast<unsigned long long*>(workspace);
    p.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + counter_bytes(d));
    p.tag = counter_tag();
  }
  p.sa_ld = lhs_scales_ld;
  p.m = m; p.n = n; p.k = k; p.kg = k / 128; p.nb = int(cdiv(n, 128));
  p.tiles_m = d.tiles_m; p.tiles_n = d.tiles_n; p.splits = d.splits; p.groups_per_split = d.gps;
  return launch(program_for(c, FP8G_JIT_DENSE, fmt, n, k), p, int64_t(d.tiles_m) * d.tiles_n * d.splits, stream);
}

int fp8_jit_grouped_gemm_contiguous(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                                    const uint8_t* rhs, const float* rhs_scales, uint16_t* out,
                                    const int32_t* m_indices, int m_total, int n, int k, int num_groups,
                                    const fp8_gemm_config* config, void* stream) {
  if (m_total < 0 || num_groups < 0) return FP8G_EINVAL;
  if (const int st = check_gemm_shape(n, k)) return st;
  if (m_total % 128 != 0) return FP8G_EUNSUPPORTED;
  if (m_total == 0 || n == 0 || num_groups == 0) return FP8G_OK;
  if (!lhs || !lhs_scales || !rhs || !rhs_scales || !out || !m_indices) return FP8G_EINVAL;
  if (!aligned16(lhs) || !aligned16(lhs_scales) || !aligned16(rhs) || !aligned16(rhs_scales) || !aligned16(out) ||
      !aligned16(m_indices))
    return FP8G_EINVAL;
  if (const int st = check_ld(lhs_scales_ld, m_total)) return st;
  fp8_gemm_config c = from_shape(kContiguousShape, 1);
  if (config) c = *config;
  apply_debug_depth(c);
  if (!valid_config(c, FP8G_JIT_CONTIGUOUS)) return FP8G_EUNSUPPORTED;
  GemmParams p{};
  p.a = lhs; p.sa = lhs_scales; p.b = rhs; p.sb = rhs_scales; p.out = out;
  p.m_indices = m_indices;
  p.sa_ld = lhs_scales_ld;
  p.m = m_total; p.n = n; p.k = k; p.kg = k / 128; p.nb = int(cdiv(n, 128));
  p.tiles_m = m_total / 128; p.tiles_n = int(cdiv(n, c.block_n)); p.splits = 1; p.groups_per_split = p.kg;
  return launch(program_for(c, FP8G_JIT_CONTIGUOUS, 0, n, k), p, int64_t(p.tiles_m) * p.tiles_n, stream);
}

int fp8_jit_grouped_gemm_masked(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                                const uint8_t* rhs, const float* rhs_scales, uint16_t* out,
                                const int32_t* masked_m, int num_groups, int max_m, int n, int k,
                                const fp8_gemm_config* config, void* stream) {
  if (num_groups < 0 || max_m < 0) return FP8G_EINVAL;
  if (const int st = check_gemm_shape(n, k)) return st;
  if (num_groups == 0 || max_m == 0 || n == 0) return FP8G_OK;
  if (!lhs || !lhs_scales || !rhs || !rhs_scales || !out || !masked_m) return FP8G_EINVAL;
  if (!aligned16(lhs) || !aligned16(lhs_scales) || !aligned16(rhs) || !aligned16(rhs_scales) || !aligned16(out) ||
      !aligned16(masked_m))
    return FP8G_EINVAL;
  if (const int st = check_ld(lhs_scales_ld, max_m)) return st;
  fp8_gemm_config c = from_shape(kMaskedShape, 1);
  if (config) c = *config;
  apply_debug_depth(c);
  if (!valid_config(c, FP8G_JIT_MASKED)) return FP8G_EUNSUPPORTED;
  GemmParams p{};
  p.a = lhs; p.sa = lhs_scales; p.b = rhs; p.sb = rhs_scales; p.out = out;
  p.masked_m = masked_m;
  p.sa_ld = lhs_scales_ld;
  p.m = max_m; p.n = n; p.k = k; p.kg = k / 128; p.nb = int(cdiv(n, 128));
  p.tiles_m = int(cdiv(max_m, c.block_m)); p.tiles_n = int(cdiv(n, c.block_n)); p.splits = 1;
  p.groups_per_split = p.kg;
  return launch(program_for(c, FP8G_JIT_MASKED, 0, n, k), p, int64_t(p.tiles_m) * p.tiles_n * num_groups, stream);
}

int fp8_jit_set_cache_dir(const char* dir) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_cache_dir = (dir && *dir) ? dir : default_cache_dir();
  return FP8G_OK;
}

int fp8_jit_get_cache_dir(char* buf, size_t len) {
  if (!buf || len == 0) return FP8G_EINVAL;
  std::lock_guard<std::mutex> lock(g_mu);
  std::snprintf(buf, len, "%s", cache_dir_locked().c_str());
  return FP8G_OK;
}

int fp8_jit_stats(long long* counts, int n) {
  if (!counts || n < 0) return FP8G_EINVAL;
  for (int i = 0; i < n && i < 5; ++i) counts[i] = g_stat[i].load();
  return FP8G_OK;
}

}  // extern "C"
